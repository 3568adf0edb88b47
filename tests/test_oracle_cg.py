"""Pins for the oracle's Clebsch-Gordan coefficients (CPU only).

The e3j paper (Appendix G.2) reconstructs the coefficients only up to
normalisation and never fixes a phase, so the oracle follows the textbook
Condon-Shortley convention (Racah's formula) plus the standard complex-to-real
change of basis.  Each test below checks it against something other than its
own formula: closed forms, an eigen-decomposition of J^2 done with numpy,
symmetry relations, orthonormality, the dot/cross products, the Gaunt identity
and rotational equivariance with Wigner-D matrices fitted from scipy's
spherical harmonics.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special as sp

from oracle import oracle as O

LMAX = 3


def triples(lmax_in=LMAX, lmax_out=2 * LMAX):
    for l1, l2 in itertools.product(range(lmax_in + 1), repeat=2):
        for L in range(abs(l1 - l2), min(l1 + l2, lmax_out) + 1):
            yield l1, l2, L


# ---------------------------------------------------------------- complex CG

def test_stretched_closed_form():
    # L = l1 + l2:  <l1 m1 l2 m2|L M>^2 = C(2l1,l1+m1) C(2l2,l2+m2) / C(2L,L+M), positive
    for l1 in range(4):
        for l2 in range(4):
            L = l1 + l2
            for m1 in range(-l1, l1 + 1):
                for m2 in range(-l2, l2 + 1):
                    M = m1 + m2
                    ref = math.sqrt(math.comb(2 * l1, l1 + m1) * math.comb(2 * l2, l2 + m2)
                                    / math.comb(2 * L, L + M))
                    assert O.cg_complex(l1, m1, l2, m2, L, M) == pytest.approx(ref, abs=1e-14)


def test_singlet_closed_form():
    # <l m l -m|0 0> = (-1)^(l-m) / sqrt(2l+1)
    for l in range(7):
        for m in range(-l, l + 1):
            ref = (-1) ** (l - m) / math.sqrt(2 * l + 1)
            assert O.cg_complex(l, m, l, -m, 0, 0) == pytest.approx(ref, abs=1e-14)


def _jops(l):
    """J_z, J_+, J_- in the |l m> basis, m = -l..l (standard ladder elements)."""
    n = 2 * l + 1
    ms = np.arange(-l, l + 1)
    jz = np.diag(ms).astype(float)
    jp = np.zeros((n, n))
    for i, m in enumerate(ms[:-1]):
        jp[i + 1, i] = math.sqrt(l * (l + 1) - m * (m + 1))
    return jz, jp, jp.T.copy()


def _cg_by_eigh(l1, l2):
    """Coupled basis of V_l1 (x) V_l2 from eigh of J^2 in every M sector.

    Phases: the top state |L L> has a positive component on m1 = l1; lower
    states are fixed so that <L M-1| J_- |L M> > 0.  Returns dict L -> array
    [2L+1, 2l1+1, 2l2+1] with entries <l1 m1 l2 m2 | L M>."""
    z1, p1, m1_ = _jops(l1)
    z2, p2, m2_ = _jops(l2)
    I1, I2 = np.eye(2 * l1 + 1), np.eye(2 * l2 + 1)
    Jz = np.kron(z1, I2) + np.kron(I1, z2)
    Jp = np.kron(p1, I2) + np.kron(I1, p2)
    Jm = np.kron(m1_, I2) + np.kron(I1, m2_)
    J2 = Jm @ Jp + Jz @ Jz + Jz
    Mdiag = np.round(np.diag(Jz)).astype(int)
    out = {}
    for L in range(abs(l1 - l2), l1 + l2 + 1):
        vecs = {}
        for M in range(L, -L - 1, -1):
            idx = np.where(Mdiag == M)[0]
            w, V = np.linalg.eigh(J2[np.ix_(idx, idx)])
            k = np.argmin(np.abs(w - L * (L + 1)))
            assert abs(w[k] - L * (L + 1)) < 1e-9
            v = np.zeros(J2.shape[0])
            v[idx] = V[:, k]
            if M == L:
                # component m1 = l1, m2 = L - l1 in the kron(V_l1, V_l2) basis
                j = (2 * l1) * (2 * l2 + 1) + (L - l1 + l2)
                if v[j] < 0:
                    v = -v
            else:
                if (vecs[M + 1] @ Jp @ v) < 0:  # <M+1|J+|M> = <M|J-|M+1>
                    v = -v
            vecs[M] = v
        blk = np.zeros((2 * L + 1, 2 * l1 + 1, 2 * l2 + 1))
        for M, v in vecs.items():
            blk[M + L] = v.reshape(2 * l1 + 1, 2 * l2 + 1)
        out[L] = blk
    return out


@pytest.mark.parametrize("l1,l2", list(itertools.product(range(LMAX + 1), repeat=2)))
def test_racah_equals_eigh_construction(l1, l2):
    ref = _cg_by_eigh(l1, l2)
    for L, blk in ref.items():
        for M in range(-L, L + 1):
            for m1 in range(-l1, l1 + 1):
                for m2 in range(-l2, l2 + 1):
                    got = O.cg_complex(l1, m1, l2, m2, L, M)
                    assert got == pytest.approx(blk[M + L, m1 + l1, m2 + l2], abs=1e-12)


def test_symmetry_relations():
    for l1, l2, L in triples():
        s = (-1) ** (l1 + l2 - L)
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                c = O.cg_complex(l1, m1, l2, m2, L, m1 + m2)
                assert O.cg_complex(l2, m2, l1, m1, L, m1 + m2) == pytest.approx(s * c, abs=1e-14)
                assert O.cg_complex(l1, -m1, l2, -m2, L, -m1 - m2) == pytest.approx(s * c, abs=1e-14)


def test_complex_orthonormality():
    for l1, l2 in itertools.product(range(LMAX + 1), repeat=2):
        rows = []
        for L in range(abs(l1 - l2), l1 + l2 + 1):
            for M in range(-L, L + 1):
                rows.append([O.cg_complex(l1, m1, l2, m2, L, M)
                             for m1 in range(-l1, l1 + 1) for m2 in range(-l2, l2 + 1)])
        U = np.array(rows)
        n = (2 * l1 + 1) * (2 * l2 + 1)
        assert U.shape == (n, n)
        np.testing.assert_allclose(U @ U.T, np.eye(n), atol=1e-13)
        np.testing.assert_allclose(U.T @ U, np.eye(n), atol=1e-13)


# ------------------------------------------------------------------- real CG

def test_umat_is_unitary():
    for l in range(7):
        U = O.umat(l)
        np.testing.assert_allclose(U @ U.conj().T, np.eye(2 * l + 1), atol=1e-14)


def test_real_blocks_orthonormal_and_nnz():
    # Frobenius norm^2 of a block = 2L+1; rows orthonormal.  nnz of the real
    # blocks for the paths that the l <= 3 configurations use.
    expected_nnz = {(0, 1, 1): 3, (1, 1, 0): 3, (1, 1, 1): 6, (1, 1, 2): 11, (1, 2, 1): 11,
                    (1, 2, 2): 16, (1, 2, 3): 21, (1, 3, 2): 21, (1, 3, 3): 26, (2, 2, 0): 5,
                    (2, 2, 1): 16, (2, 2, 2): 25, (2, 2, 3): 28, (2, 3, 1): 21, (2, 3, 2): 28,
                    (2, 3, 3): 41, (3, 3, 0): 7, (3, 3, 1): 26, (3, 3, 2): 41, (3, 3, 3): 42}
    for l1, l2, L in triples():
        T = O.cg_real(l1, l2, L)
        G = np.einsum("Mij,Nij->MN", T, T)
        np.testing.assert_allclose(G, np.eye(2 * L + 1), atol=1e-13)
        if (l1, l2, L) in expected_nnz:
            assert int((np.abs(T) > 1e-12).sum()) == expected_nnz[(l1, l2, L)]


def test_identity_paths():
    for l in range(LMAX + 1):
        T = O.cg_real(0, l, l)
        np.testing.assert_allclose(T[:, 0, :], np.eye(2 * l + 1), atol=1e-14)
        T = O.cg_real(l, 0, l)
        np.testing.assert_allclose(T[:, :, 0], np.eye(2 * l + 1), atol=1e-14)


def _real_l1(v):
    """Cartesian (x, y, z) -> real l = 1 components in m = -1, 0, 1 order (y, z, x)."""
    return np.array([v[1], v[2], v[0]])


def test_dot_and_cross_products():
    rng = np.random.default_rng(0)
    for _ in range(5):
        a, b = rng.standard_normal(3), rng.standard_normal(3)
        ra, rb = _real_l1(a), _real_l1(b)
        dot = np.einsum("Mij,i,j->M", O.cg_real(1, 1, 0), ra, rb)
        assert dot[0] == pytest.approx(-(a @ b) / math.sqrt(3), abs=1e-14)
        cr = np.einsum("Mij,i,j->M", O.cg_real(1, 1, 1), ra, rb)
        np.testing.assert_allclose(cr, _real_l1(np.cross(a, b)) / math.sqrt(2), atol=1e-14)


def test_swap_symmetry_of_equal_degree_paths():
    # l1 = l2: even paths are symmetric in (m1, m2), odd ones antisymmetric
    for l in range(1, LMAX + 1):
        for L in range(0, 2 * l + 1):
            T = O.cg_real(l, l, L)
            s = 1 if L % 2 == 0 else -1
            np.testing.assert_allclose(T, s * T.transpose(0, 2, 1), atol=1e-14)


def test_gaunt_identity():
    # For even paths the coupled product of two harmonics of the same vector
    # is a harmonic of degree L, with kappa = sqrt((2l1+1)(2l2+1)/(2L+1)) <l1 0 l2 0|L 0>.
    rng = np.random.default_rng(1)
    r = rng.standard_normal((6, 3))
    Y = O.sh(3, r)
    off = [0, 1, 4, 9]
    for l1, l2, L in triples(LMAX, LMAX):
        if (l1 + l2 + L) % 2:
            continue
        kappa = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * L + 1)) * O.cg_complex(l1, 0, l2, 0, L, 0)
        T = O.cg_real(l1, l2, L)
        v = np.einsum("Mij,ni,nj->nM", T, Y[:, off[l1]:off[l1] + 2 * l1 + 1],
                      Y[:, off[l2]:off[l2] + 2 * l2 + 1])
        np.testing.assert_allclose(v, kappa * Y[:, off[L]:off[L] + 2 * L + 1], atol=1e-12)
    # a few of those constants written out
    assert math.sqrt(3 * 3 / 5) * O.cg_complex(1, 0, 1, 0, 2, 0) == pytest.approx(math.sqrt(6 / 5))
    assert math.sqrt(3 * 3 / 1) * O.cg_complex(1, 0, 1, 0, 0, 0) == pytest.approx(-math.sqrt(3))
    assert math.sqrt(3 * 5 / 3) * O.cg_complex(1, 0, 2, 0, 1, 0) == pytest.approx(-math.sqrt(2))


def _real_sh_scipy(l, pts):
    """sqrt(4 pi) U_l Y_l^m(complex, scipy, Condon-Shortley) at unit points."""
    x, y, z = pts.T
    theta = np.arccos(np.clip(z, -1, 1))
    phi = np.arctan2(y, x)
    Yc = np.stack([sp.sph_harm_y(l, m, theta, phi) for m in range(-l, l + 1)], axis=1)
    Yr = math.sqrt(4 * math.pi) * Yc @ O.umat(l).T
    assert np.abs(Yr.imag).max() < 1e-12
    return Yr.real


def _rand_rot(rng):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q @ np.diag(np.sign(np.diag(r)))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def wigner_d(l, R, rng):
    """D^l(R) fitted by least squares from harmonics sampled on random points."""
    P = rng.standard_normal((4 * (2 * l + 1) + 8, 3))
    P /= np.linalg.norm(P, axis=1, keepdims=True)
    A = _real_sh_scipy(l, P)
    B = _real_sh_scipy(l, P @ R.T)
    D = np.linalg.lstsq(A, B, rcond=None)[0].T
    np.testing.assert_allclose(A @ D.T, B, atol=1e-10)  # fit is exact
    return D


def test_real_blocks_are_equivariant():
    rng = np.random.default_rng(2)
    R = _rand_rot(rng)
    D = {l: wigner_d(l, R, rng) for l in range(2 * LMAX + 1)}
    for l1, l2, L in triples():
        T = O.cg_real(l1, l2, L)
        lhs = np.einsum("Mij,ia,jb->Mab", T, D[l1], D[l2])
        rhs = np.einsum("MN,Nab->Mab", D[L], T)
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_real_blocks_are_real():
    # the part of U_L C (U1^dag x U2^dag) that the Re/Im rule drops is zero
    for l1, l2, L in triples():
        Cc = np.zeros((2 * L + 1, 2 * l1 + 1, 2 * l2 + 1))
        for M in range(-L, L + 1):
            for m1 in range(-l1, l1 + 1):
                for m2 in range(-l2, l2 + 1):
                    Cc[M + L, m1 + l1, m2 + l2] = O.cg_complex(l1, m1, l2, m2, L, M)
        T = np.einsum("MN,Nab,ia,jb->Mij", O.umat(L), Cc, O.umat(l1).conj(), O.umat(l2).conj())
        if (l1 + l2 + L) % 2 == 0:
            assert np.abs(T.imag).max() < 1e-13
            np.testing.assert_allclose(T.real, O.cg_real(l1, l2, L), atol=1e-13)
        else:
            assert np.abs(T.real).max() < 1e-13
            np.testing.assert_allclose(T.imag, O.cg_real(l1, l2, L), atol=1e-13)
