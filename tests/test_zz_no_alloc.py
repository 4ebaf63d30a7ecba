"""The CSR build that allocates nothing (cgtp_build_csr_order_noalloc, the
library's fixed device scratch) against cgtp_build_csr_order with a caller
workspace and against the oracle's stable sort, through the C ABI: two calls
in a row, the second on a smaller graph (the scratch keeps the first call's
contents), both CSR paths (small graphs: two launches; large graphs: the
counting sort), and the size limit."""
import ctypes

import numpy as np
import pytest

import oracle
from clebsch_gordan_tensor_cg_amd import workloads as W
from tests.gpu_util import binding

pytestmark = pytest.mark.gpu


def _graph(case):
    if case == "large_then_small":
        g = W.periodic_graph(4096, cutoff=5.0, seed=0)            # 213,738 edges: counting-sort path
        h = W.molecule_batch(100, 18, seed=0)                       # 25,710 edges: two-launch path
    else:
        g = W.molecule_batch(100, 18, seed=1)
        rs = np.random.default_rng(3)
        n = 700
        h = W.Graph(n, np.zeros((n, 3)), rs.integers(0, n, 5000).astype(np.int32),
                    rs.integers(0, n, 5000).astype(np.int32), np.zeros((5000, 3)))
    return [(g.dst, g.src, g.n_nodes), (h.dst, h.src, h.n_nodes)]


def _raw_noalloc(B, torch, key, val, n):
    """One call through the C ABI: returns perm, row_ptr, sorted_key, sorted_val, order."""
    E = key.shape[0]
    outs = [torch.full((E,), -7, dtype=torch.int32, device="cuda"),
            torch.full((n + 1,), -7, dtype=torch.int32, device="cuda"),
            torch.full((E,), -7, dtype=torch.int32, device="cuda"),
            torch.full((E,), -7, dtype=torch.int32, device="cuda"),
            torch.full((n,), -7, dtype=torch.int32, device="cuda")]
    rc = B.lib().cgtp_build_csr_order_noalloc(key.data_ptr(), val.data_ptr(), E, n, *[t.data_ptr() for t in outs],
                                              None)
    assert rc == 0, B.lib().cgtp_last_error().decode()
    return outs


@pytest.mark.parametrize("case", ["large_then_small", "small_then_smaller"])
def test_noalloc_csr_matches_workspace_call(case):
    import torch
    B = binding()
    for k, (dst, src, n) in enumerate(_graph(case)):
        print(f"noalloc csr {case} call {k}: E={len(dst)} N={n}", flush=True)
        key = torch.from_numpy(np.ascontiguousarray(dst, np.int32)).cuda()
        val = torch.from_numpy(np.ascontiguousarray(src, np.int32)).cuda()
        got = _raw_noalloc(B, torch, key, val, n)
        ref = B.cgtp_build_csr_order(key, n, val=val)
        torch.cuda.synchronize()
        g = [t.cpu().numpy() for t in got]
        r = [t.cpu().numpy() for t in ref]
        perm_o, rp_o = oracle.csr(dst, n)
        for a, b, what in zip(g[:4], r[:4], ("perm", "row_ptr", "sorted_key", "sorted_val")):
            np.testing.assert_array_equal(a, b, err_msg=what)
        np.testing.assert_array_equal(g[0], perm_o)
        np.testing.assert_array_equal(g[1], rp_o)
        np.testing.assert_array_equal(g[3], np.asarray(src)[perm_o])
        # the node order: a permutation of the rows by non-increasing length
        # (rows of 1023 or more edges tie); rows of equal length may come in
        # any order, so compare the lengths it lists with the workspace call's
        deg = np.diff(rp_o)
        assert np.array_equal(np.sort(g[4]), np.arange(n))
        np.testing.assert_array_equal(np.minimum(deg[g[4]], 1023), np.minimum(deg[r[4]], 1023))
        assert np.all(np.diff(np.minimum(deg[g[4]], 1023)) <= 0)


def test_noalloc_csr_rejects_graphs_beyond_the_scratch():
    B = binding()
    buf = (ctypes.c_int32 * 16)()
    L = B.lib()
    # 9,000,000 edges need 36 MB of scratch, more than the fixed 32 MiB: refused before any launch
    assert L.cgtp_build_csr_order_noalloc(buf, None, 9_000_000, 100, buf, buf, None, None, None, None) == -1
    assert "scratch" in L.cgtp_last_error().decode()
    assert L.cgtp_build_csr_order_noalloc(buf, None, -1, 100, buf, buf, None, None, None, None) == -1
