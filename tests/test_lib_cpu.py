"""CPU-only checks of the HIP library: it loads, exports every call that
include/cgtp.h declares, and its host-side planner agrees with the oracle
(coupling tensors, path lists, dimensions) and reports documented errors.
No GPU compute is launched here."""
import os
import re

import numpy as np
import pytest

import oracle
from clebsch_gordan_tensor_cg_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from clebsch_gordan_tensor_cg_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from clebsch_gordan_tensor_cg_amd import build
        build.build(verbose=False)
    return binding


def test_exports_every_declared_symbol(B):
    hdr = open(os.path.join(ROOT, "include", "cgtp.h")).read()
    declared = set(re.findall(r"\b(cgtp_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations found"
    L = B.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert set(B.EXPORTS) == declared
    assert "gfx950" in B.version()


def test_planner_coupling_matches_oracle(B):
    worst = 0.0
    for l1 in range(7):
        for l2 in range(7):
            for l3 in range(abs(l1 - l2), min(l1 + l2, 6) + 1):
                p = B.Plan(f"1x{l1}", f"1x{l2}", f"1x{l3}", mode="uvw", no_load=True)
                R = p.coupling(0, (2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
                worst = max(worst, np.abs(R - oracle.real_cg(l1, l2, l3)).max())
    assert worst < 1e-13, worst


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_plan_dims_and_paths_match_oracle(B, name):
    c = W.config(name)
    op = oracle.Problem(c.irreps_in1, c.irreps_in2, c.irreps_out, c.mode, c.paths, c.shared_weights)
    p = B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, c.dtype, c.shared_weights,
               no_load=True)
    assert p.paths() == op.paths
    assert (p.dim_in1, p.dim_in2, p.dim_out, p.weight_numel) == (op.dim1, op.dim2, op.dim3,
                                                                 op.weight_numel)


@pytest.mark.parametrize("name,n_paths,nnz", [("c1", 7, 37), ("c2", 10, 86), ("c3", 17, 215), ("c5", 44, 1132)])
def test_plan_dump(name, n_paths, nnz):
    """CGTP_DEBUG prints the plan: its path and CG-nonzero counts (the
    workloads' counts, and the oracle's own nonzeros of each path's real
    coupling tensor) and every kernel kind's work split, whose units cover
    every path exactly once."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from clebsch_gordan_tensor_cg_amd import binding as B, workloads as W\n"
            "c = W.config(%r)\n"
            "B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, c.dtype, c.shared_weights, "
            "no_load=True)\n" % (ROOT, name))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, CGTP_DEBUG="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    err = r.stderr
    assert f"  {n_paths} paths, {nnz} nonzeros," in err, err[-3000:]
    c = W.config(name)
    op = oracle.Problem(c.irreps_in1, c.irreps_in2, c.irreps_out, c.mode, c.paths, c.shared_weights)
    irr = lambda s: oracle.parse_irreps(s)
    a, b, o = irr(c.irreps_in1), irr(c.irreps_in2), irr(c.irreps_out)
    onz = sum(int((np.abs(oracle.real_cg(a[i].l, b[j].l, o[k].l)) > 1e-14).sum()) for i, j, k in op.paths)
    assert onz == nnz
    for line in err.splitlines():
        m = re.match(r"  path (\d+): .* (\d+) nonzeros,", line)
        if m:
            i, j, k = op.paths[int(m.group(1))]
            assert int(m.group(2)) == int((np.abs(oracle.real_cg(a[i].l, b[j].l, o[k].l)) > 1e-14).sum())
    # every kernel kind's groups cover the paths once
    kinds = re.split(r"\n  (?:forward\+backward|double backward|backward|forward): ", err)
    seen = 0
    for blk in kinds[1:]:
        paths = []
        for m in re.finditer(r"group \d+: paths \[([0-9 ]*)\]", blk):
            paths += [int(v) for v in m.group(1).split()]
        assert sorted(paths) == list(range(n_paths)), blk
        seen += 1
    assert seen >= 1


def test_generated_source_has_each_nonzero_once_per_channel_slot(B):
    c = W.config("c1")
    p = B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, c.dtype, no_load=True)
    src = p.source()
    assert "cgtp_fwd" in src and "cgtp_bwd" in src
    nnz = sum(int((np.abs(oracle.real_cg(*ls)) > 1e-14).sum())
              for ls in [(0, 0, 0), (0, 1, 1), (0, 2, 2), (1, 0, 1), (1, 1, 0), (1, 1, 2), (1, 2, 1)])
    # one FMA per nonzero into an accumulator in the forward kernel
    fwd = src[src.index("cgtp_fwd"):src.index("cgtp_bwd")]
    assert len(re.findall(r"\ba0_\d+_\d+ = fma\(", fwd)) == nnz


def test_uvw_matrix_core_source_contracts_each_nonzero_once(B, monkeypatch):
    """The uvw path-tensor kernels apply the coupling with one term per CG
    nonzero of every (path, v, k) column: the default per-pair kernel after
    its products P_i = sum_e y_e x_e,i on the matrix cores, the optional
    per-node kernel (tuning switch umma) likewise.  The per-edge kernel
    (pform=0) has no matrix-core code (its channel mixing is a library
    kernel)."""
    a, b, c = "8x0+8x1+8x2", "1x0+1x1+1x2", "12x0+12x1+12x2"
    nnz = 0
    for l1 in range(3):
        for l2 in range(3):
            for l3 in range(abs(l1 - l2), min(l1 + l2, 2) + 1):
                nnz += int((np.abs(oracle.real_cg(l1, l2, l3)) > 1e-14).sum())
    monkeypatch.setenv("CGTP_TUNE", "pform=0")
    plain = B.Plan(a, b, c, None, "uvw", "bf16", True, no_load=True).source()
    assert "__builtin_amdgcn_mfma" not in plain
    monkeypatch.setenv("CGTP_TUNE", "")
    pf = B.Plan(a, b, c, None, "uvw", "bf16", True, no_load=True).source()
    assert "__builtin_amdgcn_mfma_f32_32x32x16_bf16" in pf and "__builtin_amdgcn_permlane32_swap" in pf
    # contraction terms "c * c<half>_<tile>[<register>]", one per nonzero
    assert len(re.findall(r"[-+] 0x[0-9a-fp.+-]+f \* c[01]_\d+\[\d+\]", pf)) == nnz
    monkeypatch.setenv("CGTP_TUNE", "umma=1")
    src = B.Plan(a, b, c, None, "uvw", "bf16", True, no_load=True).source()
    assert "__builtin_amdgcn_mfma_f32_16x16x16bf16_1k" in src and "cgtp_uvw_pf" not in src
    # contraction terms "c * pr[j]", one per nonzero
    assert len(re.findall(r"[-+] 0x[0-9a-fp.+-]+f \* pr\[\d+\]", src)) == nnz


@pytest.mark.parametrize("args,code", [
    (("8x0e+", "1x0e", "8x0e"), -1),          # grammar
    (("8x0e", "1x0e", "8x1e"), -1),           # no allowed path
    (("8x0e+8x1o", "1x0e", "8x0e+4x1o"), 0),  # uvu skips the mismatched block when enumerating
    (("8x7e", "1x0e", "8x7e"), -2),           # degree above 6
    (("8x0e", "1x0", "8x0e"), 0),             # unlabelled input 2 with labelled others is allowed
    (("8x0e+8x1", "1x0e", "8x0e"), -1),       # mixed labels in one string
])
def test_plan_errors(B, args, code):
    if code == 0:
        B.Plan(*args, no_load=True)
        return
    with pytest.raises(B.CgtpError) as ei:
        B.Plan(*args, no_load=True)
    assert ei.value.code == code


def test_explicit_path_errors(B):
    with pytest.raises(B.CgtpError) as ei:
        B.Plan("8x0e+8x1o", "1x0e+1x1o", "8x0e+8x1o", paths=[(0, 1, 0)], no_load=True)  # 0e x 1o -> 0e
    assert ei.value.code == -1
    with pytest.raises(B.CgtpError) as ei:
        B.Plan("8x0e", "1x0e", "4x0e", paths=[(0, 0, 0)], no_load=True)  # uvu needs mul_out == mul_in1
    assert ei.value.code == -1
    with pytest.raises(B.CgtpError) as ei:
        B.Plan("8x0e", "1x0e", "8x0e", paths=[(0, 0, 3)], no_load=True)
    assert ei.value.code == -1


def test_compile_failure_is_reported(B, tmp_path, monkeypatch):
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))
    monkeypatch.setenv("CGTP_FAULT", "compile")
    with pytest.raises(B.CgtpError) as ei:
        B.Plan("3x0e+3x1o", "1x0e+1x1o", "3x0e+3x1o", no_load=True)
    assert ei.value.code == -3
    assert "CGTP_FAULT" in B.lib().cgtp_last_error().decode()


def test_no_load_plan_refuses_execution(B):
    """A plan made with CGTP_PLAN_NO_LOAD has no kernels on a device: every
    execution call refuses it on the host, before any launch."""
    import ctypes
    p = B.Plan("8x0e", "1x0e", "8x0e", no_load=True)
    buf = (ctypes.c_double * 64)()
    L = B.lib()
    assert L.cgtp_forward(p.handle, buf, buf, buf, 2, buf, None, 0, None) == -1
    assert "NO_LOAD" in L.cgtp_last_error().decode()
    assert L.cgtp_tp_backward(p.handle, buf, buf, buf, 2, buf, buf, None, None, buf, 512, None) == -1
    assert L.cgtp_backward(p.handle, buf, buf, buf, buf, buf, None, buf, buf, buf, 2, 2, buf, None, None, buf, 512,
                           None) == -1
    assert L.cgtp_double_backward(p.handle, buf, buf, buf, buf, None, buf, None, buf, buf, None, buf, buf, 2, 2, buf,
                                  None, None, None, buf, 512, None) == -1


def test_cache_round_trip(B, tmp_path, monkeypatch):
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))
    p1 = B.Plan("5x0e+5x1o", "1x0e+1x1o", "5x0e+5x1o", no_load=True)
    assert not p1.cached
    assert len(os.listdir(tmp_path)) == 1
    p2 = B.Plan("5x0e+5x1o", "1x0e+1x1o", "5x0e+5x1o", no_load=True)
    assert p2.cached


def test_plan_flag_combinations(B, tmp_path, monkeypatch):
    """Documented flag rules: bf16 weight storage for uvu float plans only;
    radial weights for bf16 uvw shared-weight plans whose input 2 is one SH
    row, hidden width 1..64."""
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))
    sh3 = "1x0e+1x1o+1x2e+1x3o"
    B.Plan("8x0e+8x1o", sh3, "8x0e+8x1o", bf16_weights=True, no_load=True)
    for args, kw in [
        (("8x0e", "1x0e", "8x0e", None, "uvu", "f64"), dict(bf16_weights=True)),
        (("8x0", "1x0", "8x0", None, "uvw", "bf16", True), dict(bf16_weights=True)),
        (("8x0", "1x0+1x1", "8x0+8x1", None, "uvw", "bf16", False), dict(radial_hidden=4)),   # not shared
        (("8x0", "1x0+1x1", "8x0+8x1", None, "uvw", "f32", True), dict(radial_hidden=4)),     # not bf16
        (("8x0", "2x0+1x1", "8x0+8x1", None, "uvw", "bf16", True), dict(radial_hidden=4)),    # not an SH row
        (("8x0", "1x0+1x1", "8x0+8x1", None, "uvw", "bf16", True), dict(radial_hidden=65)),   # too wide
    ]:
        with pytest.raises(B.CgtpError) as ei:
            B.Plan(*args, **kw, no_load=True)
        assert ei.value.code == -2, (args, kw)
    p = B.Plan("8x0+8x1", "1x0+1x1+1x2", "8x0+8x1", None, "uvw", "bf16", True, radial_hidden=3, no_load=True)
    # radial plans: (H+1) copies of every path along the mixing contraction
    plain = B.Plan("8x0+8x1", "1x0+1x1+1x2", "8x0+8x1", None, "uvw", "bf16", True, no_load=True)
    assert B.cgtp_workspace_bytes(p, 100) >= 4 * B.cgtp_workspace_bytes(plain, 100) - 1024


def test_graph_helper_sizes(B):
    import ctypes
    b = ctypes.c_size_t()
    assert B.lib().cgtp_node_order_workspace_bytes(100000, ctypes.byref(b)) == 0 and b.value > 0
    assert B.lib().cgtp_sparse_attention_layout_bytes(1000, 5000, ctypes.byref(b)) == 0
    # distinct columns of 63 windows: at most the edges plus 16 padding slots per window
    assert b.value >= 4 * (5000 + 16 * 63) + 2 * (5000 + 16 * 63)
    assert B.lib().cgtp_node_order_workspace_bytes(-1, ctypes.byref(b)) == -1
    assert B.lib().cgtp_sparse_attention_layout_bytes(-1, 5, ctypes.byref(b)) == -1


def test_csr_argument_errors(B):
    """cgtp_build_csr / cgtp_build_csr_order reject bad sizes, NULL buffers and
    short workspaces before any launch (no GPU needed to reach the checks)."""
    import ctypes
    L = B.lib()
    b = ctypes.c_size_t()
    assert L.cgtp_csr_workspace_bytes(1000, 50, ctypes.byref(b)) == 0
    need = b.value
    key = (ctypes.c_int32 * 4)()
    out = (ctypes.c_int32 * 64)()
    ws = (ctypes.c_uint8 * max(need, 1))()
    for fn, extra in ((L.cgtp_build_csr, ()), (L.cgtp_build_csr_order, (out,))):
        # negative sizes
        assert fn(key, None, -1, 50, out, out, None, None, *extra, ws, need, None) == -1
        # keys but no perm
        assert fn(key, None, 1000, 50, None, out, None, None, *extra, ws, need, None) == -1
        # values wanted without a value array
        assert fn(key, None, 1000, 50, out, out, None, out, *extra, ws, need, None) == -1
        # workspace too small
        assert fn(key, None, 1000, 50, out, out, None, None, *extra, ws, need - 1, None) == -1
        assert "cgtp_build_csr" in L.cgtp_last_error().decode()


def test_sh_from_vectors_needs_sh_row_plan(B):
    """cgtp_conv_forward_vec refuses plans whose input 2 is not one SH row
    before any device work (checked on the host)."""
    import ctypes
    p = B.Plan("8x0e+8x1o", "2x0e+1x1o", "8x0e+8x1o", no_load=True)
    buf = (ctypes.c_double * 64)()
    rc = B.lib().cgtp_conv_forward_vec(p.handle, buf, buf, None, buf, buf, buf, None, 2, 1, buf, None, 0, None)
    assert rc == -2
    assert "SH row" in B.lib().cgtp_last_error().decode()


def test_workspace_query(B):
    """cgtp_workspace_bytes: one size for every execution call of a plan;
    argument errors before any device contact."""
    import ctypes
    L = B.lib()
    b = ctypes.c_size_t()
    c = W.config("c2")
    p = B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, c.dtype, no_load=True)
    assert L.cgtp_workspace_bytes(None, 10, 10, ctypes.byref(b)) == -1
    assert L.cgtp_workspace_bytes(p.handle, -1, 10, ctypes.byref(b)) == -1
    assert L.cgtp_workspace_bytes(p.handle, 10, -1, ctypes.byref(b)) == -1
    assert L.cgtp_workspace_bytes(p.handle, 10, 10, None) == -1
    # uvu: the backward's per-edge x-messages (E x dim1 floats) dominate
    E = 213738
    n = B.cgtp_workspace_bytes(p, 4096, E)
    assert n >= E * p.dim_in1 * 4 + E * 3 * 4
    assert B.cgtp_workspace_bytes(p, 4096, 2 * E) > n
    # single product: its backward counts each item as one edge
    assert B.cgtp_workspace_bytes(p, 1000, 0) == B.cgtp_workspace_bytes(p, 1000, 1000)
    # uvw: the path tensors of every item (bf16), at least
    c5 = W.config("c5")
    q = B.Plan(c5.irreps_in1, c5.irreps_in2, c5.irreps_out, c5.paths, c5.mode, c5.dtype, c5.shared_weights,
               no_load=True)
    assert B.cgtp_workspace_bytes(q, 1800, 0) >= 1800 * 2 * 32 * 1132 // 16


def test_sh_helpers_argument_errors(B):
    """cgtp_sh and cgtp_sh_vjp_forces check sizes, NULL buffers, dtype and
    degree on the host before any launch."""
    import ctypes
    L = B.lib()
    buf = (ctypes.c_double * 64)()
    F32, F64, BF16 = 0, 1, 2
    assert L.cgtp_sh(3, F32, buf, None, -1, buf, None) == -1
    assert L.cgtp_sh(3, F32, None, None, 4, buf, None) == -1
    assert L.cgtp_sh(3, 7, buf, None, 4, buf, None) == -2          # unknown dtype
    assert L.cgtp_sh(7, F32, buf, None, 4, buf, None) == -2        # degree above 6
    assert L.cgtp_sh(3, F32, None, None, 0, None, None) == 0       # nothing to do
    # vjp / forces: bf16 is not provided; negative sizes; forces need both CSRs
    assert L.cgtp_sh_vjp_forces(3, BF16, buf, None, buf, buf, buf, buf, 2, 2, buf, buf, None, 0, None) == -2
    assert L.cgtp_sh_vjp_forces(3, F32, buf, None, buf, buf, buf, buf, -1, 2, buf, buf, None, 0, None) == -1
    assert L.cgtp_sh_vjp_forces(3, F32, buf, None, buf, None, buf, buf, 2, 2, buf, buf, None, 0, None) == -1
    assert L.cgtp_sh_vjp_forces(3, F32, None, None, buf, buf, buf, buf, 2, 2, buf, buf, None, 0, None) == -1
    # forces without g_vec need 3 E elements of workspace
    assert L.cgtp_sh_vjp_forces(3, F64, buf, None, buf, buf, buf, buf, 2, 2, None, buf, buf, 47, None) == -1
    assert L.cgtp_sh_vjp_forces(7, F64, buf, None, buf, buf, buf, buf, 2, 2, buf, buf, None, 0, None) == -2
    # neither output: nothing to do
    assert L.cgtp_sh_vjp_forces(3, F32, buf, None, buf, None, None, None, 2, 2, None, None, None, 0, None) == 0


def test_csr_transpose_canonical_argument_errors(B):
    """Sizes and NULL buffers are checked on the host before any launch."""
    import ctypes
    L = B.lib()
    buf = (ctypes.c_int32 * 16)()
    assert L.cgtp_build_csr_transpose_canonical(buf, buf, -1, 3, buf, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(buf, buf, 4, -1, buf, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(buf, buf, 1 << 31, 3, buf, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(None, buf, 4, 3, buf, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(buf, None, 4, 3, buf, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(buf, buf, 4, 3, None, buf, None) == -1
    assert L.cgtp_build_csr_transpose_canonical(buf, buf, 4, 3, buf, None, None) == -1


def test_stream_probe_argument_errors(B):
    """The bandwidth probe checks its kind, size and alignment on the host
    before any launch; an empty size does nothing."""
    import ctypes
    L = B.lib()
    buf = (ctypes.c_double * 8)()
    base = ctypes.addressof(buf)
    a = base + (-base % 16)        # a 16-byte aligned address inside buf
    assert L.cgtp_stream_probe(3, a, a, 16, None) == -1              # unknown kind
    assert L.cgtp_stream_probe(-1, a, a, 16, None) == -1
    assert L.cgtp_stream_probe(2, a, a, 24, None) == -1              # not a multiple of 16
    assert L.cgtp_stream_probe(2, a + 4, a, 16, None) == -1          # misaligned source
    assert L.cgtp_stream_probe(1, None, a + 8, 16, None) == -1       # misaligned destination
    assert L.cgtp_stream_probe(0, None, a, 16, None) == -1           # a read needs a source
    assert L.cgtp_stream_probe(1, None, None, 16, None) == -1        # every kind needs dst
    assert L.cgtp_stream_probe(2, a, a, 0, None) == 0                # nothing to move
    with pytest.raises(ValueError):
        B.cgtp_stream_probe("scan", None, None)


def test_binding_rejects_bad_arguments(B):
    """The binding checks shape, dtype, contiguity and device of every tensor
    before it calls the library, so a short buffer, a wrong dtype or a host
    tensor never reaches a kernel as a raw pointer."""
    import torch
    c = W.config("c2")
    p = B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, c.dtype, no_load=True)
    N, E = 5, 7
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    f32 = lambda *s: torch.zeros(*s)
    x, sh, w, g = f32(N, p.dim_in1), f32(E, p.dim_in2), f32(E, p.weight_numel), f32(N, p.dim_out)
    src, rp, sperm, srp = i32(E), i32(N + 1), i32(E), i32(N + 1)
    ok = dict(x=x, sh=sh, w=w, src=src, dst_row_ptr=rp)

    def fwd(**kw):
        a = dict(ok, **kw)
        return B.cgtp_conv_forward(p, a["x"], a["sh"], a["w"], a["src"], a["dst_row_ptr"],
                                   node_order=a.get("node_order"), out=a.get("out"))

    with pytest.raises(ValueError, match="sh: expected shape"):
        fwd(sh=f32(E - 1, p.dim_in2))
    with pytest.raises(ValueError, match="w: expected shape"):
        fwd(w=f32(E, p.weight_numel - 1))
    with pytest.raises(ValueError, match="dst_row_ptr: expected shape"):
        fwd(dst_row_ptr=i32(N))
    with pytest.raises(ValueError, match="node_order: expected shape"):
        fwd(node_order=i32(N + 1))
    with pytest.raises(ValueError, match="out: expected shape"):
        fwd(out=f32(N, p.dim_out + 1))
    with pytest.raises(TypeError, match="x: expected torch.float32"):
        fwd(x=torch.zeros(N, p.dim_in1, dtype=torch.float64))
    with pytest.raises(TypeError, match="src: expected torch.int32"):
        fwd(src=torch.zeros(E, dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        fwd(w=f32(p.weight_numel, E).t())
    with pytest.raises(ValueError, match="on cpu"):
        fwd()
    with pytest.raises(ValueError, match="g_out: expected shape"):
        B.cgtp_backward(p, x, sh, w, src, rp, srp, sperm, f32(N, p.dim_out - 1))
    with pytest.raises(ValueError, match="src_perm: expected shape"):
        B.cgtp_backward(p, x, sh, w, src, rp, srp, i32(E + 1), g)
    with pytest.raises(ValueError, match="gg_sh: expected shape"):
        B.cgtp_double_backward(p, x, None, w, g, None, f32(E + 1, p.dim_in2), None, src, rp, srp, sperm)
    with pytest.raises(ValueError, match="vec: expected shape"):
        B.cgtp_conv_forward_vec(p, x, f32(E + 1, 3), None, w, src, rp)
    with pytest.raises(TypeError, match="vec: expected torch.float32"):
        B.cgtp_conv_forward_vec(p, x, torch.zeros(E, 3, dtype=torch.float64), None, w, src, rp)
    with pytest.raises(ValueError, match="g_sh: expected shape"):
        B.cgtp_sh_vjp_forces(3, f32(E, 3), None, f32(E, 15), rp, srp, sperm)
    with pytest.raises(ValueError, match="dst_row_ptr is required"):
        B.cgtp_sh_vjp_forces(3, f32(E, 3), None, f32(E, 16), None, srp, sperm)
    with pytest.raises(ValueError, match="on cpu"):
        B.cgtp_sh(3, f32(E, 3))
    # FP64 plans want float64 everywhere (vectors included)
    p64 = B.Plan(c.irreps_in1, c.irreps_in2, c.irreps_out, c.paths, c.mode, "f64", no_load=True)
    with pytest.raises(TypeError, match="x: expected torch.float64"):
        B.cgtp_conv_forward(p64, x, sh.double(), w.double(), src, rp)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises: there is no CPU fallback."""
    from clebsch_gordan_tensor_cg_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libcgtp.so"))
    with pytest.raises(RuntimeError, match="is not built"):
        binding.lib()
    with pytest.raises(RuntimeError, match="is not built"):
        binding.Plan("8x0e", "1x0e", "8x0e", no_load=True)
    with pytest.raises(RuntimeError, match="is not built"):
        binding.cgtp_csr_workspace_bytes(10, 10)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU: asked for more it exits with a message
    and a non-zero status before it touches any device."""
    import json
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parents[1]
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], cwd=root, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus_requested"] == 2 and "one GPU" in msg["error"]
