"""FP64 CPU oracle for the CG tensor product and its graph convolution.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this package, and this package imports nothing from the product.

It follows the plain definitions (complex CG from the Racah formula, real
basis change, component-normalised real spherical harmonics, explicit-loop
tensor product, convolution, adjoints, forces), as described by
"An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep Networks"
(abstract: CG tensor product fused with a graph convolution, its gradient
and the higher derivatives needed for forces) and by the SE(3)-Transformer
page's TFN section (degree d has 2d+1 components; contributions to one
output degree are summed).  The arithmetic lives in ``cgtp_oracle.c``;
this module parses irreps, lists paths and marshals numpy arrays.

Readings taken where the pages are silent (each is also listed in the
design notes): no path or irrep normalisation factors; plain-sum
aggregation; real-basis phase fixed by the basis change below (odd
l1+l2+l3 keeps the imaginary part); r_e = pos[dst] - pos[src].
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cgtp_oracle.c")
# CGTP_ORACLE_LIB: another build of the same source to load instead (the
# sanitizer test's); it is never rebuilt here
_LIB = os.environ.get("CGTP_ORACLE_LIB") or os.path.join(_HERE, "libcgtp_oracle.so")


def build_oracle(force: bool = False) -> str:
    """Compile the C oracle with gcc (host only)."""
    if os.environ.get("CGTP_ORACLE_LIB"):
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build_oracle()
        L = ctypes.CDLL(_LIB)
        d, i32, i64, vp = ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.orc_cg_complex.restype = d
        L.orc_cg_complex.argtypes = [i32] * 6
        L.orc_real_cg.restype = i32
        L.orc_real_cg.argtypes = [i32, i32, i32, vp]
        L.orc_sh.restype = None
        L.orc_sh.argtypes = [i32, i64, vp, vp]
        L.orc_sh_jacobian.restype = None
        L.orc_sh_jacobian.argtypes = [i32, i64, vp, vp]
        L.orc_tp_forward.restype = i32
        L.orc_tp_forward.argtypes = [vp, i32, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp]
        L.orc_tp_backward.restype = i32
        L.orc_tp_backward.argtypes = [vp, i32, i32, i64, i64, i64, i64, i64, i64,
                                      vp, vp, vp, vp, vp, vp, vp]
        L.orc_conv_forward.restype = i32
        L.orc_conv_forward.argtypes = [vp, i32, i32, i64, i64, vp, vp, i64, i64, i64, i64,
                                       vp, vp, vp, vp]
        L.orc_conv_backward.restype = i32
        L.orc_conv_backward.argtypes = [vp, i32, i32, i64, i64, vp, vp, i64, i64, i64, i64,
                                        i64, vp, vp, vp, vp, vp, vp, vp]
        L.orc_forces.restype = i32
        L.orc_forces.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
        L.orc_force_loss_cotangent.restype = i32
        L.orc_force_loss_cotangent.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
        L.orc_csr.restype = i32
        L.orc_csr.argtypes = [vp, i64, i64, vp, vp]
        L.orc_set_threads.restype = i32
        L.orc_set_threads.argtypes = [i32]
        L.orc_sparse_attention.restype = i32
        L.orc_sparse_attention.argtypes = [i64, i64, i64, vp, vp, i32, i32, d, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# --------------------------------------------------------------------------
# Irreps and paths (O(3) labels "MULxLp"; a degree-l block has 2l+1 entries)
# --------------------------------------------------------------------------

_TERM = re.compile(r"^\s*(\d+)\s*x\s*(\d+)\s*([eo]?)\s*$")


@dataclass(frozen=True)
class Irrep:
    mul: int
    l: int
    p: int  # +1 even, -1 odd, 0 no parity label

    @property
    def dim(self) -> int:
        return 2 * self.l + 1


def parse_irreps(s: str) -> list[Irrep]:
    out = []
    for term in s.split("+"):
        m = _TERM.match(term)
        if not m:
            raise ValueError(f"bad irreps term {term!r} in {s!r}")
        mul, l, par = int(m.group(1)), int(m.group(2)), m.group(3)
        out.append(Irrep(mul, l, {"e": 1, "o": -1, "": 0}[par]))
    labelled = {ir.p != 0 for ir in out}
    if len(labelled) > 1:
        raise ValueError(f"mixed parity-labelled and unlabelled irreps in {s!r}")
    return out


def irreps_dim(irreps) -> int:
    return sum(ir.mul * ir.dim for ir in irreps)


def irreps_offsets(irreps) -> list[int]:
    offs, o = [], 0
    for ir in irreps:
        offs.append(o)
        o += ir.mul * ir.dim
    return offs


def path_allowed(a: Irrep, b: Irrep, c: Irrep) -> bool:
    if not (abs(a.l - b.l) <= c.l <= a.l + b.l):
        return False
    if a.p and b.p and c.p and a.p * b.p != c.p:
        return False
    return True


def all_paths(in1, in2, out, mode: str) -> list[tuple[int, int, int]]:
    """Every allowed (i1, i2, i3), i1 outer, then i2, then i3."""
    res = []
    for i1, a in enumerate(in1):
        for i2, b in enumerate(in2):
            for i3, c in enumerate(out):
                if not path_allowed(a, b, c):
                    continue
                if mode == "uvu" and c.mul != a.mul:
                    continue
                res.append((i1, i2, i3))
    return res


_PATH_DT = np.dtype([("l1", np.int32), ("l2", np.int32), ("l3", np.int32),
                     ("mul1", np.int32), ("mul2", np.int32), ("mul3", np.int32),
                     ("off1", np.int64), ("off2", np.int64), ("off3", np.int64),
                     ("woff", np.int64)])


class Problem:
    """Irreps, path list and weight layout of one tensor product."""

    def __init__(self, irreps_in1: str, irreps_in2: str, irreps_out: str, mode: str = "uvu",
                 paths=None, shared_weights: bool = False):
        if mode not in ("uvu", "uvw"):
            raise ValueError(mode)
        self.in1, self.in2, self.out = (parse_irreps(irreps_in1), parse_irreps(irreps_in2),
                                        parse_irreps(irreps_out))
        self.mode = mode
        self.shared_weights = shared_weights
        if paths is None:
            paths = all_paths(self.in1, self.in2, self.out, mode)
        self.paths = [tuple(p) for p in paths]
        o1, o2, o3 = (irreps_offsets(self.in1), irreps_offsets(self.in2),
                      irreps_offsets(self.out))
        rows, woff = [], 0
        for (i1, i2, i3) in self.paths:
            a, b, c = self.in1[i1], self.in2[i2], self.out[i3]
            if not path_allowed(a, b, c):
                raise ValueError(f"forbidden path {(i1, i2, i3)}")
            if mode == "uvu" and c.mul != a.mul:
                raise ValueError(f"uvu path {(i1, i2, i3)} needs mul_out == mul_in1")
            rows.append((a.l, b.l, c.l, a.mul, b.mul, c.mul, o1[i1], o2[i2], o3[i3], woff))
            woff += a.mul * b.mul * (c.mul if mode == "uvw" else 1)
        self.table = np.array(rows, dtype=_PATH_DT)
        self.dim1, self.dim2, self.dim3 = (irreps_dim(self.in1), irreps_dim(self.in2),
                                           irreps_dim(self.out))
        self.weight_numel = woff
        self._mode = 0 if mode == "uvu" else 1

    @property
    def wrow(self) -> int:
        return 0 if self.shared_weights else self.weight_numel

    # ---------------- single tensor product (items independent) ----------
    def tp_forward(self, x, y, w):
        x, y, w = _f64(x), _f64(y), _f64(w)
        B = x.shape[0]
        out = np.empty((B, self.dim3))
        rc = lib().orc_tp_forward(_p(self.table), len(self.paths), self._mode, B, self.dim1,
                                  self.dim2, self.dim3, self.wrow, _p(x), _p(y), _p(w), _p(out))
        assert rc == 0
        return out

    def tp_backward(self, x, y, w, g):
        x, y, w, g = _f64(x), _f64(y), _f64(w), _f64(g)
        B = x.shape[0]
        gx, gy = np.empty_like(x), np.empty_like(y)
        gw = np.empty(self.weight_numel) if self.shared_weights else np.empty_like(w)
        rc = lib().orc_tp_backward(_p(self.table), len(self.paths), self._mode, B, self.dim1,
                                   self.dim2, self.dim3, self.wrow, self.weight_numel,
                                   _p(x), _p(y), _p(w), _p(g), _p(gx), _p(gy), _p(gw))
        assert rc == 0
        return gx, gy, gw

    # ---------------- graph convolution ----------------------------------
    def conv_forward(self, x, sh, w, src, dst, n_nodes):
        x, sh, w, src, dst = _f64(x), _f64(sh), _f64(w), _i32(src), _i32(dst)
        out = np.empty((n_nodes, self.dim3))
        rc = lib().orc_conv_forward(_p(self.table), len(self.paths), self._mode, n_nodes,
                                    len(src), _p(src), _p(dst), self.dim1, self.dim2,
                                    self.dim3, self.wrow, _p(x), _p(sh), _p(w), _p(out))
        assert rc == 0
        return out

    def conv_backward(self, x, sh, w, src, dst, g_out, need=("x", "sh", "w")):
        x, sh, w, src, dst, g_out = (_f64(x), _f64(sh), _f64(w), _i32(src), _i32(dst),
                                     _f64(g_out))
        n_nodes = x.shape[0]
        gx = np.empty_like(x) if "x" in need else None
        gy = np.empty_like(sh) if "sh" in need else None
        gw = None
        if "w" in need:
            gw = np.empty(self.weight_numel) if self.shared_weights else np.empty_like(w)
        rc = lib().orc_conv_backward(_p(self.table), len(self.paths), self._mode, n_nodes,
                                     len(src), _p(src), _p(dst), self.dim1, self.dim2,
                                     self.dim3, self.wrow, self.weight_numel, _p(x), _p(sh),
                                     _p(w), _p(g_out), _p(gx), _p(gy), _p(gw))
        assert rc == 0
        return gx, gy, gw

    def conv_double_backward(self, x, sh, w, src, dst, g_out, gg_x=None, gg_sh=None,
                             gg_w=None):
        """Second derivatives by trilinearity of f(x, y, w).

        With cotangents (a_x, a_y, a_w) on the backward's outputs
        (g_x, g_y, g_w), S = <g, f(a_x,y,w) + f(x,a_y,w) + f(x,y,a_w)>, so
          dS/dg = f(a_x,y,w) + f(x,a_y,w) + f(x,y,a_w)
          dS/dx = fx*(g; a_y, w) + fx*(g; y, a_w)
          dS/dy = fy*(g; a_x, w) + fy*(g; x, a_w)
          dS/dw = fw*(g; a_x, y) + fw*(g; x, a_y)
        where fx*, fy*, fw* are the backward's adjoints.  Absent cotangents
        are zero.  Returns (d_g_out, d_x, d_sh, d_w).
        """
        n = x.shape[0]
        z = lambda a: np.zeros_like(_f64(a))
        ax = z(x) if gg_x is None else _f64(gg_x)
        ay = z(sh) if gg_sh is None else _f64(gg_sh)
        aw = z(w) if gg_w is None else _f64(gg_w)
        dg = (self.conv_forward(ax, sh, w, src, dst, n) + self.conv_forward(x, ay, w, src, dst, n)
              + self.conv_forward(x, sh, aw, src, dst, n))
        gx1, _, gw1 = self.conv_backward(x, ay, w, src, dst, g_out)     # a_y terms
        gx2, gy2, _ = self.conv_backward(x, sh, aw, src, dst, g_out)    # a_w terms
        _, gy3, gw3 = self.conv_backward(ax, sh, w, src, dst, g_out)    # a_x terms
        d_x = gx1 + gx2
        d_sh = gy3 + gy2
        d_w = gw3 + gw1
        return dg, d_x, d_sh, d_w


# --------------------------------------------------------------------------
# Stand-alone pieces
# --------------------------------------------------------------------------

def set_threads(n: int) -> int:
    """OpenMP threads of the oracle's loops (0 keeps the current count);
    returns the count in effect.  Timing only: results do not change."""
    return int(lib().orc_set_threads(int(n)))


def cg_complex(j1, m1, j2, m2, J, M) -> float:
    return lib().orc_cg_complex(j1, m1, j2, m2, J, M)


def real_cg(l1, l2, l3) -> np.ndarray:
    R = np.empty((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    if lib().orc_real_cg(l1, l2, l3, _p(R)) != 0:
        raise ValueError((l1, l2, l3))
    return R


def spherical_harmonics(lmax: int, r) -> np.ndarray:
    r = _f64(r).reshape(-1, 3)
    Y = np.empty((r.shape[0], (lmax + 1) ** 2))
    lib().orc_sh(lmax, r.shape[0], _p(r), _p(Y))
    return Y


def sh_jacobian(lmax: int, r) -> np.ndarray:
    r = _f64(r).reshape(-1, 3)
    J = np.empty((r.shape[0], (lmax + 1) ** 2, 3))
    lib().orc_sh_jacobian(lmax, r.shape[0], _p(r), _p(J))
    return J


def forces(lmax, n_nodes, src, dst, r, g_sh) -> np.ndarray:
    src, dst, r, g_sh = _i32(src), _i32(dst), _f64(r), _f64(g_sh)
    F = np.empty((n_nodes, 3))
    rc = lib().orc_forces(lmax, n_nodes, len(src), _p(src), _p(dst), _p(r), _p(g_sh), _p(F))
    assert rc == 0
    return F


def force_loss_cotangent(lmax, n_nodes, src, dst, r, F) -> np.ndarray:
    """gg_sh = dL/dg_sh for L = 1/2 sum |F|^2."""
    src, dst, r, F = _i32(src), _i32(dst), _f64(r), _f64(F)
    gg = np.empty((len(src), (lmax + 1) ** 2))
    rc = lib().orc_force_loss_cotangent(lmax, n_nodes, len(src), _p(src), _p(dst), _p(r),
                                        _p(F), _p(gg))
    assert rc == 0
    return gg


def csr(key, n_nodes):
    """Stable sort of edge ids by key -> (perm, row_ptr), both int32."""
    key = _i32(key)
    perm = np.empty(len(key), np.int32)
    row_ptr = np.empty(n_nodes + 1, np.int32)
    rc = lib().orc_csr(_p(key), len(key), n_nodes, _p(perm), _p(row_ptr))
    assert rc == 0
    return perm, row_ptr


def sparse_attention(q, k, v, src, dst, n_rows, scale=None):
    """Graph sparse attention, per head (Fused3S abstract: SDDMM, softmax,
    SpMM).  q [n_rows][H][d], k and v [n_cols][H][d]; edges src -> dst in
    any order; scale defaults to 1/sqrt(d).  Rows without edges are zero."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    src, dst = _i32(src), _i32(dst)
    H, d = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((n_rows, H, d))
    rc = lib().orc_sparse_attention(n_rows, k.shape[0], len(src), _p(src), _p(dst), H, d, float(scale),
                                    _p(q), _p(k), _p(v), _p(out))
    assert rc == 0
    return out


# --------------------------------------------------------------------------
# Per-edge radial weights ("Faster training and inference with NVIDIA's
# open-source SE(3)-Transformer", fused keys and values section: the radial
# profile inside a TFN layer is a fully connected network).  Reading: one
# hidden layer of width H on the edge length r, SiLU activation, a linear
# output layer with bias producing the layer's whole weight row:
#   phi_h(r) = silu(a_h r + c_h),  silu(z) = z / (1 + e^-z)
#   W_e = w[0] + sum_{h=1..H} phi_h(|r_e|) w[h]        (w: [H+1][weight_numel])
# The edge's weights then enter the tensor product as per-item weights.
# --------------------------------------------------------------------------
def radial_hidden(r, radial):
    """phi [E][H] for edge lengths r [E]; radial = [2][H] (a, then c)."""
    r = _f64(r).reshape(-1, 1)
    radial = _f64(radial)
    z = r * radial[0][None, :] + radial[1][None, :]
    return z / (1.0 + np.exp(-z))


def radial_weights(r, radial, w):
    """Per-edge weight rows W [E][weight_numel] from the radial network."""
    w = _f64(w)
    phi = radial_hidden(r, radial)
    return w[0][None, :] + phi @ w[1:]


def conv_forward_radial(prob, x, sh, r, radial, w, src, dst, n_nodes):
    """Convolution whose per-edge weights come from the radial network of
    the edge lengths r (prob must hold per-item weights)."""
    assert not prob.shared_weights
    return prob.conv_forward(x, sh, radial_weights(r, radial, w), src, dst, n_nodes)
