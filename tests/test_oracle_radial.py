"""Pins of the oracle's radial weights (oracle/radial.py): the Bessel basis
against its orthonormality on [0, r_c] with weight d^2 and its closed values,
SiLU against closed values, the MLP against one-hot closed forms, linearity,
rotation invariance and an independently written generator, and the
backward against central differences, the bilinear identity in W2 and the
radial direction of the edge-vector gradient."""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from oracle import radial as R

RC = 5.0


def test_bessel_basis_orthonormal_with_weight_d2():
    # int_0^rc B_n(d) B_m(d) d^2 dd = (2/rc) int_0^rc sin(n pi d/rc) sin(m pi d/rc) dd = delta_nm
    xg, wg = np.polynomial.legendre.leggauss(200)
    d = 0.5 * RC * (xg + 1.0)
    B = R.bessel_basis(d, RC, 8)
    G = (B * (0.5 * RC * wg * d ** 2)[:, None]).T @ B
    np.testing.assert_allclose(G, np.eye(8), atol=1e-12)


def test_bessel_basis_closed_values_and_limit():
    B = R.bessel_basis(np.array([RC / 2]), RC, 4)[0]
    a = np.sqrt(2.0 / RC) * 2.0 / RC
    np.testing.assert_allclose(B, [a, 0.0, -a, 0.0], atol=1e-15)
    b0 = R.bessel_basis(np.array([0.0]), RC, 8)[0]
    b_eps = R.bessel_basis(np.array([1e-7]), RC, 8)[0]
    np.testing.assert_allclose(b0, np.sqrt(2.0 / RC) * np.pi * np.arange(1, 9) / RC, rtol=1e-15)
    np.testing.assert_allclose(b_eps, b0, rtol=1e-10)


def test_bessel_basis_derivative_by_differences():
    d = np.array([0.3, 1.1, 2.5, 4.9])
    h = 1e-6
    fd = (R.bessel_basis(d + h, RC, 8) - R.bessel_basis(d - h, RC, 8)) / (2 * h)
    np.testing.assert_allclose(R.bessel_basis_deriv(d, RC, 8), fd, rtol=1e-7, atol=1e-9)


def test_silu_values_and_derivative():
    assert R.silu(0.0) == 0.0
    assert R.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert R.silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-15)
    t = np.linspace(-6, 6, 25)
    h = 1e-6
    np.testing.assert_allclose(R.silu_deriv(t), (R.silu(t + h) - R.silu(t - h)) / (2 * h),
                               rtol=1e-8, atol=1e-10)


def test_mlp_one_hot_closed_form():
    rng = np.random.default_rng(0)
    ev = rng.standard_normal((9, 3))
    d = np.linalg.norm(ev, axis=1)
    n, k, j = 2, 5, 7
    W1 = np.zeros((8, 64))
    W1[n, k] = 1.0
    W2 = np.zeros((64, 12))
    W2[k, j] = 1.0
    w = R.radial_mlp(ev, RC, W1, W2)
    b = np.sqrt(2.0 / RC) * np.sin((n + 1) * np.pi * d / RC) / d
    expect = np.zeros_like(w)
    expect[:, j] = b / (1.0 + np.exp(-b))
    # the other hidden units see pre-activation 0 and silu(0) = 0
    np.testing.assert_allclose(w, expect, rtol=1e-14, atol=1e-15)


def test_mlp_linear_in_w2_and_rotation_invariant():
    rng = np.random.default_rng(1)
    ev = rng.standard_normal((20, 3)) * 2
    W1 = rng.standard_normal((8, 64)) / np.sqrt(8)
    Wa, Wb = rng.standard_normal((2, 64, 30)) / 8
    np.testing.assert_allclose(R.radial_mlp(ev, RC, W1, Wa + Wb),
                               R.radial_mlp(ev, RC, W1, Wa) + R.radial_mlp(ev, RC, W1, Wb),
                               rtol=1e-12, atol=1e-13)
    q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    np.testing.assert_allclose(R.radial_mlp(ev @ q.T, RC, W1, Wa), R.radial_mlp(ev, RC, W1, Wa),
                               rtol=1e-12, atol=1e-13)


def test_mlp_matches_the_input_generator():
    # the water workload's weights were produced by an independently written
    # fp64 evaluation of the same reading (input generation); same W1, W2
    g = S.random_graph(60, 8.0, 4.0, seed=3)
    P, C = 3, 4
    ref = S.radial_mlp_weights(g.evec, 4.0, P, C, seed=5)
    W1 = S.normal((8, 64), 5, S.TAG_W1).astype(np.float64) / np.sqrt(8.0)
    W2 = S.normal((64, P * C), 5, S.TAG_W2).astype(np.float64) / np.sqrt(64.0)
    got = R.radial_mlp(g.evec, 4.0, W1, W2).reshape(-1, P, C)
    np.testing.assert_allclose(got, ref, rtol=2e-6, atol=1e-6)  # ref is stored as float32


def test_mlp_backward_by_differences_and_identities():
    rng = np.random.default_rng(2)
    ev = rng.standard_normal((6, 3)) * 1.5
    W1 = rng.standard_normal((8, 64)) / np.sqrt(8)
    W2 = rng.standard_normal((64, 10)) / 8
    dw = rng.standard_normal((6, 10))
    dW1, dW2, dvec = R.radial_mlp_backward(ev, RC, W1, W2, dw)
    loss = lambda e, a, b: np.vdot(dw, R.radial_mlp(e, RC, a, b))
    # w is linear in W2: <dW2, W2> = <dw, w>
    assert np.vdot(dW2, W2) == pytest.approx(loss(ev, W1, W2), rel=1e-12)
    # the weights depend on |r| only: the gradient is radial
    np.testing.assert_allclose(np.cross(dvec, ev), 0.0, atol=1e-12)
    h = 1e-6
    for arr, grad, k in ((W1, dW1, 1), (W2, dW2, 2), (ev, dvec, 0)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p, args_m = [ev, W1, W2], [ev, W1, W2]
            args_p[k], args_m[k] = ap, am
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-8)


def test_conv_forward_radial_equals_conv_with_computed_weights_and_samples():
    p = S.make_conv("tiny")
    g = p.graph
    d = O.Desc(p.x_irreps, p.y_irreps, p.out_irreps, p.channels)
    P = O.num_paths(d)
    rng = np.random.default_rng(4)
    W1 = rng.standard_normal((8, 64)) / np.sqrt(8)
    W2 = rng.standard_normal((64, P * p.channels)) / 8
    full = R.conv_forward_radial(d, g.rowptr, g.sender, g.evec, p.x, 3.0, W1, W2)
    w = R.radial_mlp(g.evec, 3.0, W1, W2).reshape(-1, P, p.channels)
    np.testing.assert_array_equal(full, O.conv_forward(d, g.rowptr, g.sender, p.x, w, evec=g.evec))
    rows = np.array([5, 0, 63, 17, 5])
    part = R.conv_forward_radial(d, g.rowptr, g.sender, g.evec, p.x, 3.0, W1, W2, rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-13)
