"""Pins for the oracle's coupling tensors and spherical harmonics.

Nothing here re-types the oracle's formulas: the oracle is checked against
sympy's exact Clebsch-Gordan coefficients, scipy's complex spherical
harmonics, closed forms, orthogonality, the Gaunt product rule and
rotation equivariance.
"""
import math

import numpy as np
import pytest
import sympy
from scipy.special import eval_legendre, sph_harm_y
from sympy.physics.wigner import clebsch_gordan

import oracle

rng = np.random.default_rng(1234)


def _sympy_cg(j1, m1, j2, m2, J, M):
    return float(clebsch_gordan(j1, j2, J, m1, m2, M))


@pytest.mark.parametrize("lmax", [4])
def test_complex_cg_matches_sympy(lmax):
    for j1 in range(lmax + 1):
        for j2 in range(lmax + 1):
            for J in range(abs(j1 - j2), j1 + j2 + 1):
                for m1 in range(-j1, j1 + 1):
                    for m2 in range(-j2, j2 + 1):
                        M = m1 + m2
                        if abs(M) > J:
                            continue
                        a = oracle.cg_complex(j1, m1, j2, m2, J, M)
                        b = _sympy_cg(j1, m1, j2, m2, J, M)
                        assert abs(a - b) < 1e-14, (j1, m1, j2, m2, J, M, a, b)


def test_complex_cg_matches_sympy_high_l_sample():
    for _ in range(150):
        j1, j2 = rng.integers(0, 7, size=2)
        J = int(rng.integers(abs(j1 - j2), j1 + j2 + 1))
        m1 = int(rng.integers(-j1, j1 + 1))
        m2 = int(rng.integers(-j2, j2 + 1))
        if abs(m1 + m2) > J:
            continue
        assert abs(oracle.cg_complex(int(j1), m1, int(j2), m2, J, m1 + m2)
                   - _sympy_cg(int(j1), m1, int(j2), m2, J, m1 + m2)) < 1e-13


def test_real_cg_closed_forms():
    # l (x) l -> 0 is (-1)^l delta / sqrt(2l+1)
    for l in range(7):
        R = oracle.real_cg(l, l, 0)[:, :, 0]
        np.testing.assert_allclose(R, (-1) ** l * np.eye(2 * l + 1) / math.sqrt(2 * l + 1),
                                   atol=1e-14)
    # 0 (x) l -> l and l (x) 0 -> l are the identity
    for l in range(7):
        np.testing.assert_allclose(oracle.real_cg(0, l, l)[0], np.eye(2 * l + 1), atol=1e-14)
        np.testing.assert_allclose(oracle.real_cg(l, 0, l)[:, 0, :], np.eye(2 * l + 1),
                                   atol=1e-14)
    # 1 (x) 1 -> 1 is the cross product / sqrt 2 (components in y,z,x order,
    # which is a cyclic relabelling, so the Levi-Civita tensor keeps its sign)
    eps = np.zeros((3, 3, 3))
    for (i, j, k), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[i, j, k] = s
    np.testing.assert_allclose(oracle.real_cg(1, 1, 1), eps / math.sqrt(2), atol=1e-14)


def _triples(lmax):
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                yield l1, l2, l3


def test_real_cg_orthonormal_and_complete():
    lmax = 5
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            blocks = []
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                R = oracle.real_cg(l1, l2, l3).reshape(-1, 2 * l3 + 1)
                np.testing.assert_allclose(R.T @ R, np.eye(2 * l3 + 1), atol=1e-13)
                blocks.append(R)
            B = np.concatenate(blocks, axis=1)   # square (2l1+1)(2l2+1)
            np.testing.assert_allclose(B @ B.T, np.eye(B.shape[0]), atol=1e-13)


def test_real_cg_swap_symmetry():
    for l1, l2, l3 in _triples(5):
        A = oracle.real_cg(l1, l2, l3)
        B = oracle.real_cg(l2, l1, l3)
        np.testing.assert_allclose(B, (-1) ** (l1 + l2 - l3) * A.transpose(1, 0, 2), atol=1e-13)


def _rand_dirs(n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def _scipy_real_sh(lmax, r):
    """Component-normalised real SH from scipy's complex (C-S phased) ones."""
    r = r / np.linalg.norm(r, axis=1, keepdims=True)
    theta = np.arccos(np.clip(r[:, 2], -1, 1))
    phi = np.mod(np.arctan2(r[:, 1], r[:, 0]), 2 * np.pi)
    out = np.zeros((len(r), (lmax + 1) ** 2))
    for l in range(lmax + 1):
        for m in range(-l, l + 1):
            Y = sph_harm_y(l, abs(m), theta, phi) * math.sqrt(4 * math.pi)
            if m > 0:
                v = math.sqrt(2) * (-1) ** m * Y.real
            elif m < 0:
                v = math.sqrt(2) * (-1) ** m * Y.imag
            else:
                v = Y.real
            out[:, l * l + m + l] = v
    return out


def test_sh_matches_scipy():
    r = rng.standard_normal((200, 3)) * 3.0
    np.testing.assert_allclose(oracle.spherical_harmonics(6, r), _scipy_real_sh(6, r),
                               atol=1e-12, rtol=0)


def test_sh_closed_form_l1_and_norm():
    r = rng.standard_normal((50, 3))
    Y = oracle.spherical_harmonics(4, r)
    u = r / np.linalg.norm(r, axis=1, keepdims=True)
    np.testing.assert_allclose(Y[:, 1:4], math.sqrt(3) * u[:, [1, 2, 0]], atol=1e-14)
    np.testing.assert_allclose(Y[:, 0], 1.0, atol=1e-15)
    for l in range(5):
        np.testing.assert_allclose((Y[:, l * l:(l + 1) ** 2] ** 2).sum(1), 2 * l + 1, rtol=1e-13)


def test_sh_addition_theorem():
    a, b = _rand_dirs(40), _rand_dirs(40)
    Ya, Yb = oracle.spherical_harmonics(6, a), oracle.spherical_harmonics(6, b)
    cos = (a * b).sum(1)
    for l in range(7):
        s = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose((Ya[:, s] * Yb[:, s]).sum(1),
                                   (2 * l + 1) * eval_legendre(l, cos), atol=1e-12)


def test_gaunt_product_rule_links_cg_and_sh():
    """sum_ij R_ijk Y_l1,i(r) Y_l2,j(r) = c Y_l3,k(r), with
    c = sqrt((2l1+1)(2l2+1)/(2l3+1)) <l1 0 l2 0 | l3 0> (sympy, exact)."""
    r = _rand_dirs(30)
    Y = _scipy_real_sh(6, r)
    for l1, l2, l3 in _triples(4):
        if l1 + l2 > 6:
            continue
        R = oracle.real_cg(l1, l2, l3)
        Y1, Y2, Y3 = (Y[:, l * l:(l + 1) ** 2] for l in (l1, l2, l3))
        lhs = np.einsum("ijk,ni,nj->nk", R, Y1, Y2)
        c = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * float(
            clebsch_gordan(l1, l2, l3, 0, 0, 0))
        np.testing.assert_allclose(lhs, c * Y3, atol=1e-12)
    # two values the closed forms fix
    assert math.isclose(math.sqrt(9) * float(clebsch_gordan(1, 1, 0, 0, 0, 0)), -math.sqrt(3))


def random_rotation(rs):
    q = rs.standard_normal(4)
    q /= np.linalg.norm(q)
    a, b, c, d = q
    return np.array([[a*a+b*b-c*c-d*d, 2*(b*c-a*d), 2*(b*d+a*c)],
                     [2*(b*c+a*d), a*a-b*b+c*c-d*d, 2*(c*d-a*b)],
                     [2*(b*d-a*c), 2*(c*d+a*b), a*a-b*b-c*c+d*d]])


def wigner_d(lmax, Rot, npts=80):
    """D^l with Y(Rot p) = D^l Y(p), fitted by least squares on scipy SH."""
    p = _rand_dirs(npts)
    Y0 = _scipy_real_sh(lmax, p)
    Y1 = _scipy_real_sh(lmax, p @ Rot.T)
    Ds = []
    for l in range(lmax + 1):
        s = slice(l * l, (l + 1) ** 2)
        X, *_ = np.linalg.lstsq(Y0[:, s], Y1[:, s], rcond=None)
        Ds.append(X.T)
    return Ds


def test_wigner_d_fit_sanity():
    rs = np.random.default_rng(7)
    A, B = random_rotation(rs), random_rotation(rs)
    DA, DB, DAB = wigner_d(4, A), wigner_d(4, B), wigner_d(4, A @ B)
    perm = [1, 2, 0]
    np.testing.assert_allclose(DA[1], A[np.ix_(perm, perm)], atol=1e-10)
    for l in range(5):
        np.testing.assert_allclose(DA[l] @ DA[l].T, np.eye(2 * l + 1), atol=1e-10)
        np.testing.assert_allclose(DA[l] @ DB[l], DAB[l], atol=1e-10)


def test_real_cg_equivariant():
    rs = np.random.default_rng(11)
    Rot = random_rotation(rs)
    D = wigner_d(6, Rot)
    for l1, l2, l3 in _triples(3):
        R = oracle.real_cg(l1, l2, l3)
        x = rs.standard_normal(2 * l1 + 1)
        y = rs.standard_normal(2 * l2 + 1)
        lhs = np.einsum("ijk,i,j->k", R, D[l1] @ x, D[l2] @ y)
        rhs = D[l3] @ np.einsum("ijk,i,j->k", R, x, y)
        np.testing.assert_allclose(lhs, rhs, atol=1e-10)


def test_sh_jacobian_finite_difference_and_radial():
    r = rng.standard_normal((40, 3)) * 2.0
    J = oracle.sh_jacobian(6, r)
    h = 1e-6
    for c in range(3):
        d = np.zeros(3)
        d[c] = h
        fd = (oracle.spherical_harmonics(6, r + d) - oracle.spherical_harmonics(6, r - d)) / (2 * h)
        np.testing.assert_allclose(J[:, :, c], fd, atol=2e-7)
    # Y depends on direction only: J r = 0
    np.testing.assert_allclose(np.einsum("nkc,nc->nk", J, r), 0.0, atol=1e-12)
