"""GPU parity of the fused graph sparse attention (SDDMM, softmax, SpMM) in
both forms -- 16-row windows on the matrix cores, and the row form on the
VALU -- against the FP64 oracle on the same bf16-rounded inputs."""
import numpy as np
import pytest

import oracle
from clebsch_gordan_tensor_cg_amd import workloads as W
from tests.gpu_util import assert_close, binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    return binding()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    return t


FORMS = ["windows", "rows"]


def _attend(B, torch, form, q, k, v, col, rp_d, n_cols, n_edges):
    if form == "rows":
        return B.cgtp_sparse_attention_rows(q, k, v, col, rp_d)
    layout = B.cgtp_sparse_attention_prepare(col, rp_d, n_cols)
    return B.cgtp_sparse_attention(q, k, v, rp_d, n_edges, layout)


def _run(B, torch, src, dst, n_rows, n_cols, H, D, seed, name, form="windows"):
    rs = np.random.default_rng(seed)
    q, k, v = (W.normal(rs, (n, H, D), "bf16") for n in (n_rows, n_cols, n_cols))
    perm, rp = oracle.csr(dst, n_rows)
    ref = oracle.sparse_attention(q, k, v, src, dst, n_rows)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
    print(f"attention {form} {name} rows={n_rows} E={len(src)} H={H} D={D}", flush=True)
    rp_d = torch.from_numpy(rp).cuda()
    col = torch.from_numpy(src[perm].astype(np.int32)).cuda()
    out = _attend(B, torch, form, bf(q), bf(k), bf(v), col, rp_d, n_cols, len(src))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    empty = np.setdiff1d(np.arange(n_rows), dst)
    assert np.all(got[empty] == 0.0)
    assert_close(got.reshape(n_rows, -1), ref.reshape(n_rows, -1), "bf16", name)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("H,D", [(1, 16), (4, 64), (5, 32), (3, 128), (16, 16), (6, 16)])
def test_attention_small_ragged(B, torch, H, D, form):
    rs = np.random.default_rng(H * 100 + D)
    n_rows, n_cols = 77, 90                          # ragged last window, empty rows
    src = rs.integers(0, n_cols, 900)
    dst = rs.integers(0, n_rows, 900)
    dst[dst == 10] = 11
    key = np.unique(np.stack([dst, src], 1), axis=0)     # no repeated (row, column)
    dst, src = key[:, 0].astype(np.int32), key[:, 1].astype(np.int32)
    _run(B, torch, src, dst, n_rows, n_cols, H, D, 1, "small", form)


@pytest.mark.parametrize("form", FORMS)
def test_attention_hub_row_several_batches(B, torch, form):
    """One row with 5000 distinct columns: several LDS batches continue the
    same running softmax."""
    rs = np.random.default_rng(7)
    n_rows, n_cols = 40, 6000
    hub_src = rs.permutation(n_cols)[:5000]
    src = np.concatenate([hub_src, rs.integers(0, n_cols, 300)])
    dst = np.concatenate([np.full(5000, 3), rs.integers(0, n_rows, 300)])
    key = np.unique(np.stack([dst, src], 1), axis=0)
    _run(B, torch, key[:, 1].astype(np.int32), key[:, 0].astype(np.int32), n_rows, n_cols, 2, 32, 8, "hub", form)


@pytest.mark.parametrize("form", FORMS)
def test_attention_molecule_batch(B, torch, form):
    g = W.molecule_batch(100, 18, cutoff=5.0, seed=0)
    _run(B, torch, g.src, g.dst, g.n_nodes, g.n_nodes, 8, 16, 2, "molecules", form)


@pytest.mark.parametrize("form", FORMS)
def test_attention_water_box(B, torch, form):
    g = W.periodic_graph(4096, cutoff=5.0, seed=0)
    _run(B, torch, g.src, g.dst, g.n_nodes, g.n_nodes, 8, 32, 3, "water box", form)


@pytest.mark.parametrize("form", FORMS)
def test_attention_ignores_out_of_range_columns(B, torch, form):
    rs = np.random.default_rng(9)
    n_rows, n_cols, H, D = 20, 30, 2, 16
    q, k, v = (W.normal(rs, (n, H, D), "bf16") for n in (n_rows, n_cols, n_cols))
    rp = np.concatenate([[0], np.cumsum(np.r_[[3, 3], np.zeros(n_rows - 2, int)])]).astype(np.int32)
    col = np.array([1, 45, 2, -4, 7, 7 + 1], np.int32)      # 45 and -4 are out of range
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
    rp_d = torch.from_numpy(rp).cuda()
    out = _attend(B, torch, form, bf(q), bf(k), bf(v), torch.from_numpy(col).cuda(), rp_d, n_cols, len(col))
    torch.cuda.synchronize()
    ref = oracle.sparse_attention(q, k, v, np.array([1, 2, 7, 8]), np.array([0, 0, 1, 1]), n_rows)
    assert_close(out.cpu().numpy().reshape(n_rows, -1), ref.reshape(n_rows, -1), "bf16", "out of range")
