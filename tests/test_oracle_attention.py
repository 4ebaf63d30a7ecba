"""Pins of the oracle's graph sparse attention ("Fused3S: Fast Sparse
Attention on Tensor Cores", abstract: SDDMM, softmax, SpMM) against other
formulations and closed forms."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _graph(rs, n_rows, n_cols, n_edges):
    pairs = set()
    while len(pairs) < n_edges:
        pairs.add((int(rs.integers(n_cols)), int(rs.integers(n_rows))))
    src, dst = np.array(sorted(pairs)).T
    return src.astype(np.int32), dst.astype(np.int32)


def _dense(q, k, v, src, dst, n_rows, scale):
    """Dense masked formulation: S = scale Q K^T with -inf off the edges,
    softmax along rows, O = P V (numpy matmul), per head."""
    H = q.shape[1]
    out = np.zeros((n_rows, H, q.shape[2]))
    mask = np.zeros((n_rows, k.shape[0]), bool)
    mask[dst, src] = True
    for h in range(H):
        S = scale * q[:, h, :] @ k[:, h, :].T
        S = np.where(mask, S, -np.inf)
        has = mask.any(axis=1)
        P = np.zeros_like(S)
        P[has] = softmax(S[has], axis=1)
        out[:, h, :] = P @ v[:, h, :]
    return out


@pytest.mark.parametrize("H,d", [(1, 4), (3, 16)])
def test_attention_equals_dense_masked_softmax(H, d):
    rs = np.random.default_rng(H * 10 + d)
    n_rows, n_cols = 23, 31
    src, dst = _graph(rs, n_rows, n_cols, 150)
    q, k, v = (rs.standard_normal((n, H, d)) for n in (n_rows, n_cols, n_cols))
    got = oracle.sparse_attention(q, k, v, src, dst, n_rows)
    ref = _dense(q, k, v, src, dst, n_rows, 1.0 / np.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # rows without edges are zero
    empty = np.setdiff1d(np.arange(n_rows), dst)
    assert np.all(got[empty] == 0.0)


def test_attention_single_neighbour_and_uniform_cases():
    rs = np.random.default_rng(1)
    q, k, v = rs.standard_normal((4, 2, 8)), rs.standard_normal((6, 2, 8)), rs.standard_normal((6, 2, 8))
    # row 0: one neighbour -> its value row exactly
    src, dst = np.array([3, 1, 2, 5]), np.array([0, 1, 1, 1])
    out = oracle.sparse_attention(q, k, v, src, dst, 4)
    np.testing.assert_array_equal(out[0], v[3])
    # zero queries (or zero scale): the plain mean of the neighbours' values
    out0 = oracle.sparse_attention(np.zeros_like(q), k, v, src, dst, 4)
    np.testing.assert_allclose(out0[1], v[[1, 2, 5]].mean(axis=0), rtol=1e-14, atol=1e-15)
    outs = oracle.sparse_attention(q, k, v, src, dst, 4, scale=0.0)
    np.testing.assert_allclose(outs[1], out0[1], rtol=1e-14, atol=1e-15)


def test_attention_invariances():
    rs = np.random.default_rng(2)
    n_rows, n_cols, H, d = 17, 19, 2, 8
    src, dst = _graph(rs, n_rows, n_cols, 90)
    q, k, v = (rs.standard_normal((n, H, d)) for n in (n_rows, n_cols, n_cols))
    base = oracle.sparse_attention(q, k, v, src, dst, n_rows)
    # a key shift common to all columns shifts each row's scores by a constant
    c = rs.standard_normal((1, H, d))
    np.testing.assert_allclose(oracle.sparse_attention(q, k + c, v, src, dst, n_rows), base, rtol=1e-10, atol=1e-12)
    # edge order does not matter
    p = rs.permutation(len(src))
    np.testing.assert_allclose(oracle.sparse_attention(q, k, v, src[p], dst[p], n_rows), base, rtol=1e-13, atol=1e-14)
    # outputs are convex combinations of the neighbours' values
    for i in np.unique(dst):
        nb = v[src[dst == i]]
        assert np.all(base[i] <= nb.max(axis=0) + 1e-12) and np.all(base[i] >= nb.min(axis=0) - 1e-12)
