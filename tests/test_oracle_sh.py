"""Pins for the oracle's real spherical harmonics (CPU only).

The e3j paper leaves the normalisation c_l open (Appendix G.1 Eq.20) and
notes that real harmonics fix only |m|; the oracle uses component
normalisation with m = -l..l and the standard real combination of the
Condon-Shortley complex harmonics.  Pins: scipy's complex harmonics mapped
through the same change of basis, the norm sum_m Y^2 = 2l+1, the value on the
z axis, parity, scale invariance and harmonicity of r^l Y_l.
"""
import math

import numpy as np
import pytest
import scipy.special as sp

from oracle import oracle as O

OFF = [0, 1, 4, 9, 16]


def unit(rng, n):
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_against_scipy_complex_harmonics():
    rng = np.random.default_rng(0)
    P = unit(rng, 50)
    Y = O.sh(3, P)
    x, y, z = P.T
    theta, phi = np.arccos(np.clip(z, -1, 1)), np.arctan2(y, x)
    for l in range(4):
        Yc = np.stack([sp.sph_harm_y(l, m, theta, phi) for m in range(-l, l + 1)], axis=1)
        ref = math.sqrt(4 * math.pi) * Yc @ O.umat(l).T
        assert np.abs(ref.imag).max() < 1e-12
        np.testing.assert_allclose(Y[:, OFF[l]:OFF[l + 1]], ref.real, atol=1e-12)


def test_l1_is_the_unit_vector():
    rng = np.random.default_rng(1)
    P = unit(rng, 10)
    Y = O.sh(1, P)
    np.testing.assert_allclose(Y[:, 1:4], math.sqrt(3) * P[:, [1, 2, 0]], atol=1e-15)


def test_component_normalisation():
    rng = np.random.default_rng(2)
    Y = O.sh(3, unit(rng, 100))
    for l in range(4):
        np.testing.assert_allclose((Y[:, OFF[l]:OFF[l + 1]] ** 2).sum(1), 2 * l + 1, rtol=1e-13)


def test_z_axis():
    Y = O.sh(3, np.array([[0.0, 0.0, 2.5]]))[0]
    for l in range(4):
        e = np.zeros(2 * l + 1)
        e[l] = math.sqrt(2 * l + 1)
        np.testing.assert_allclose(Y[OFF[l]:OFF[l + 1]], e, atol=1e-14)


def test_parity_and_scale():
    rng = np.random.default_rng(3)
    P = rng.standard_normal((20, 3))
    Y, Yn, Ys = O.sh(3, P), O.sh(3, -P), O.sh(3, 7.3 * P)
    for l in range(4):
        sl = slice(OFF[l], OFF[l + 1])
        np.testing.assert_allclose(Yn[:, sl], (-1) ** l * Y[:, sl], atol=1e-14)
        np.testing.assert_allclose(Ys[:, sl], Y[:, sl], atol=1e-14)


def test_harmonic_polynomials():
    # r^l Y_l(r/|r|) has zero Laplacian (central differences, fp64)
    rng = np.random.default_rng(4)
    h = 1e-3
    for p in rng.standard_normal((5, 3)):
        def f(q):
            r = np.linalg.norm(q)
            Y = O.sh(3, q[None])[0]
            return np.concatenate([r ** l * Y[OFF[l]:OFF[l + 1]] for l in range(4)])
        lap = -6 * f(p)
        for k in range(3):
            e = np.zeros(3)
            e[k] = h
            lap = lap + f(p + e) + f(p - e)
        lap /= h * h
        np.testing.assert_allclose(lap, 0, atol=1e-5)


def test_rotation_acts_linearly_within_each_degree():
    # Y_l(R r) = D^l(R) Y_l(r) with one matrix for every point (fit on some
    # points, predict the others)
    rng = np.random.default_rng(5)
    q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    A, B = unit(rng, 40), unit(rng, 10)
    YA, YAr = O.sh(3, A), O.sh(3, A @ q.T)
    YB, YBr = O.sh(3, B), O.sh(3, B @ q.T)
    for l in range(4):
        sl = slice(OFF[l], OFF[l + 1])
        D = np.linalg.lstsq(YA[:, sl], YAr[:, sl], rcond=None)[0]
        np.testing.assert_allclose(YB[:, sl] @ D, YBr[:, sl], atol=1e-12)
        np.testing.assert_allclose(D @ D.T, np.eye(2 * l + 1), atol=1e-12)


def test_zero_vector():
    Y = O.sh(3, np.zeros((1, 3)))[0]
    assert Y[0] == 1.0 and np.all(Y[1:] == 0.0)


def test_rejects_unsupported_degree():
    with pytest.raises(ValueError):
        O.sh(9, np.ones((1, 3)))
