"""Pins of the oracle at degrees 4..8 (the tensor products and convolutions
of e3j B.1, Figs 5-7, run to L = 8): the general harmonics against scipy's
complex harmonics through the change of basis, their norm, z-axis values,
parity, harmonicity and rotation behaviour, and against the closed-form
polynomials at l <= 3; the Racah coefficients against a numpy
eigen-decomposition of J^2; the real blocks' orthonormality and rotation
equivariance (Wigner-D fitted from scipy), and the Gaunt identity linking
the harmonics and the coefficients."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_cg import _cg_by_eigh, _rand_rot, _real_sh_scipy, wigner_d

LH = 8  # highest degree pinned
HI = range(4, LH + 1)
OFF = [l * l for l in range(LH + 2)]


def unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_general_harmonics_against_scipy():
    rng = np.random.default_rng(40)
    P = unit(rng, 60)
    Y = O.sh(LH, P)
    for l in range(LH + 1):
        np.testing.assert_allclose(Y[:, OFF[l]:OFF[l + 1]], _real_sh_scipy(l, P), atol=1e-11,
                                   err_msg=f"l={l}")


def test_general_construction_equals_closed_forms_at_low_degree():
    rng = np.random.default_rng(41)
    P = rng.standard_normal((25, 3)) * 3
    Y = O.sh(3, P)
    for l in range(4):
        np.testing.assert_allclose(O.sh_general(l, P), Y[:, OFF[l]:OFF[l + 1]], atol=1e-13)


def test_high_degree_norm_axis_parity_scale():
    rng = np.random.default_rng(42)
    P = rng.standard_normal((40, 3))
    Y, Yn, Ys = O.sh(LH, P), O.sh(LH, -P), O.sh(LH, 0.37 * P)
    Z = O.sh(LH, np.array([[0.0, 0.0, 1.7]]))[0]
    for l in HI:
        sl = slice(OFF[l], OFF[l + 1])
        np.testing.assert_allclose((Y[:, sl] ** 2).sum(1), 2 * l + 1, rtol=1e-12)
        np.testing.assert_allclose(Yn[:, sl], (-1) ** l * Y[:, sl], atol=1e-12)
        np.testing.assert_allclose(Ys[:, sl], Y[:, sl], atol=1e-12)
        e = np.zeros(2 * l + 1)
        e[l] = math.sqrt(2 * l + 1)
        np.testing.assert_allclose(Z[sl], e, atol=1e-12)


def test_high_degree_harmonic_polynomials():
    # r^l Y_l(r/|r|) has zero Laplacian (fourth-order central differences:
    # the second-order stencil's h^2 error is too large at degree 6; the
    # fourth-order one's h^4 error grows as l^6, hence the small step)
    rng = np.random.default_rng(43)
    h = 2e-3
    for p in rng.standard_normal((3, 3)):
        def f(q):
            r = np.linalg.norm(q)
            Y = O.sh(LH, q[None])[0]
            return np.concatenate([r ** l * Y[OFF[l]:OFF[l + 1]] for l in HI])
        lap = -90 * f(p)
        for k in range(3):
            e = np.zeros(3)
            e[k] = h
            lap = lap + 16 * (f(p + e) + f(p - e)) - (f(p + 2 * e) + f(p - 2 * e))
        np.testing.assert_allclose(lap / (12 * h * h), 0,
                                   atol=1e-5 * max(1.0, np.abs(f(p)).max()))


@pytest.mark.parametrize("l1,l2", [(l1, l2) for l1, l2 in itertools.product(range(LH + 1), repeat=2)
                                   if max(l1, l2) >= 4])
def test_racah_equals_eigh_construction_high_degree(l1, l2):
    ref = _cg_by_eigh(l1, l2)
    for L, blk in ref.items():
        for M in range(-L, L + 1):
            for m1 in range(-l1, l1 + 1):
                m2 = M - m1
                if abs(m2) > l2:
                    continue
                got = O.cg_complex(l1, m1, l2, m2, L, M)
                assert got == pytest.approx(blk[M + L, m1 + l1, m2 + l2], abs=1e-11)


def _triples_hi():
    for l1, l2 in itertools.product(range(LH + 1), repeat=2):
        for L in range(abs(l1 - l2), min(l1 + l2, LH) + 1):
            if max(l1, l2, L) >= 4:
                yield l1, l2, L


def test_real_blocks_orthonormal_high_degree():
    for l1, l2, L in _triples_hi():
        T = O.cg_real(l1, l2, L).reshape(2 * L + 1, -1)
        np.testing.assert_allclose(T @ T.T, np.eye(2 * L + 1), atol=1e-11, err_msg=str((l1, l2, L)))


def test_real_blocks_equivariant_high_degree():
    rng = np.random.default_rng(44)
    R = _rand_rot(rng)
    D = {l: wigner_d(l, R, rng) for l in range(LH + 1)}
    for l1, l2, L in _triples_hi():
        T = O.cg_real(l1, l2, L)
        lhs = np.einsum("Mij,ia,jb->Mab", T, D[l1], D[l2])
        rhs = np.einsum("MN,Nab->Mab", D[L], T)
        np.testing.assert_allclose(lhs, rhs, atol=1e-9, err_msg=str((l1, l2, L)))


def test_gaunt_identity_high_degree():
    # even paths couple two harmonics of one vector into a harmonic of degree
    # L: kappa = sqrt((2l1+1)(2l2+1)/(2L+1)) <l1 0 l2 0|L 0>
    rng = np.random.default_rng(45)
    r = rng.standard_normal((5, 3))
    Y = O.sh(LH, r)
    for l1, l2, L in _triples_hi():
        if (l1 + l2 + L) % 2:
            continue
        kappa = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * L + 1)) * \
            O.cg_complex(l1, 0, l2, 0, L, 0)
        T = O.cg_real(l1, l2, L)
        v = np.einsum("Mij,ni,nj->nM", T, Y[:, OFF[l1]:OFF[l1 + 1]], Y[:, OFF[l2]:OFF[l2 + 1]])
        np.testing.assert_allclose(v, kappa * Y[:, OFF[L]:OFF[L + 1]], atol=1e-10,
                                   err_msg=str((l1, l2, L)))


def test_zero_vector_high_degree():
    Y = O.sh(LH, np.zeros((1, 3)))[0]
    assert Y[0] == 1.0 and np.all(Y[1:] == 0.0)


# ------------------------------------------- harmonics gradient, degrees 4..8

def test_sh_grad_fd_matches_closed_form_partials():
    # the finite-difference gradient reproduces the closed-form one to l = 3
    rng = np.random.default_rng(60)
    v = rng.standard_normal((40, 3)) * rng.uniform(0.2, 5.0, (40, 1))
    dY = rng.standard_normal((40, 16))
    a, b = O.sh_grad_fd(3, v, dY), O.sh_grad(3, v, dY)
    assert np.abs(a - b).max() <= 1e-8 * np.abs(b).max()


@pytest.mark.parametrize("L", [6, 8])
def test_sh_grad_fd_high_degree_properties(L):
    # the harmonics depend on the direction only: the gradient is orthogonal
    # to r and scales as 1/|r|; a single component's gradient matches the
    # derivative of the Legendre form along a tangent direction
    rng = np.random.default_rng(61)
    n, dy = 30, (L + 1) ** 2
    v = rng.standard_normal((n, 3))
    dY = rng.standard_normal((n, dy))
    g = O.sh_grad_fd(L, v, dY)
    assert np.abs((g * v).sum(1)).max() <= 1e-8 * np.abs(g).max()
    g3 = O.sh_grad_fd(L, 3.0 * v, dY)
    assert np.abs(3.0 * g3 - g).max() <= 1e-8 * np.abs(g).max()
    # d/dphi of the m = +L component: Y_LL ~ sin^L(theta) cos(L phi), so its
    # derivative along e_phi is -L Y_L,-L / (|r| sin theta)
    u = v / np.linalg.norm(v, axis=1, keepdims=True)
    e_phi = np.stack([-u[:, 1], u[:, 0], np.zeros(n)], 1)
    e_phi /= np.linalg.norm(e_phi, axis=1, keepdims=True)
    sel = np.zeros((n, dy))
    sel[:, L * L + 2 * L] = 1.0  # (l, m) = (L, L)
    d = (O.sh_grad_fd(L, u, sel) * e_phi).sum(1)
    sin_t = np.sqrt(u[:, 0] ** 2 + u[:, 1] ** 2)
    Y = O.sh(L, u)
    np.testing.assert_allclose(d, -L * Y[:, L * L] / sin_t, rtol=1e-7, atol=1e-8)


def test_sh_grad_fd_zero_vector():
    g = O.sh_grad_fd(5, np.zeros((2, 3)), np.ones((2, 36)))
    assert np.all(g == 0.0)
