"""Helpers for the GPU parity tests: tolerances, CSR permutations computed
by the oracle, and the library handle."""
import os

import numpy as np
import pytest

import oracle

# Tolerances of the parity bar, applied per output tensor as
#   max_i |a_i - r_i| / (|r_i| + RMS(r)) <= tol
TOL = {"f32": 1e-5, "f64": 1e-12, "bf16": 2e-2}


def rel_err(a, r) -> float:
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.abs(r) + rms
    if rms == 0.0:
        return float(np.abs(a - r).max())
    return float((np.abs(a - r) / den).max())


def assert_close(a, r, dtype, what=""):
    e = rel_err(a, r)
    assert e <= TOL[dtype], f"{what}: rel err {e:.3e} > {TOL[dtype]:.0e}"
    return e


def binding():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from clebsch_gordan_tensor_cg_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from clebsch_gordan_tensor_cg_amd import build
        build.build(verbose=False)
    return B


class GraphArrays:
    """Canonical-order graph plus the CSR orders computed by the oracle."""

    def __init__(self, src, dst, n_nodes):
        self.src = np.asarray(src, np.int32)
        self.dst = np.asarray(dst, np.int32)
        self.n = n_nodes
        self.E = len(self.src)
        self.perm, self.row_ptr = oracle.csr(self.dst, n_nodes)      # dst order
        self.src_d = self.src[self.perm]                              # src per dst-ordered edge
        self.dst_d = self.dst[self.perm]
        self.src_perm, self.src_row_ptr = oracle.csr(self.src_d, n_nodes)

    def dev(self, torch, device="cuda"):
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return dict(src=t(self.src_d), dst=t(self.dst_d), dst_row_ptr=t(self.row_ptr),
                    src_row_ptr=t(self.src_row_ptr), src_perm=t(self.src_perm))


def to_dev(torch, a, dtype):
    import torch as _t
    td = {"f32": _t.float32, "f64": _t.float64, "bf16": _t.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(td)
