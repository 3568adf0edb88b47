"""Pins of the oracle's per-irrep channel mixing (e3j A.3 Eq.5 with the
equivariant mixing tensor W^{km}_{k'm'} = W^k_{k'} delta_{mm'} between blocks
of equal degree and parity).

Independent checks: numpy's einsum on block slices, the identity map,
rotation equivariance with Wigner-D matrices fitted from the harmonics,
parity selection and the summation over input blocks of one type.
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_conv import _block_rotate, _rot


def _offsets(irreps):
    o, out = 0, []
    for l, _ in irreps:
        out.append(o)
        o += 2 * l + 1
    return out


def _pairs(ins, outs):
    return [(i, o) for i in range(len(ins)) for o in range(len(outs))
            if ins[i] == outs[o]]


def _einsum_linear(ins, outs, x, W):
    rows, _, cin = x.shape
    cout = W.shape[-1]
    dout = sum(2 * l + 1 for l, _ in outs)
    y = np.zeros((rows, dout, cout))
    io, oo = _offsets(ins), _offsets(outs)
    for n, (i, o) in enumerate(_pairs(ins, outs)):
        d = 2 * ins[i][0] + 1
        y[:, oo[o]:oo[o] + d] += np.einsum("rmk,kc->rmc", x[:, io[i]:io[i] + d], W[n])
    return y


@pytest.mark.parametrize("ins,outs,cin,cout", [
    ([(0, 1), (1, -1), (2, 1), (3, -1)], [(0, 1), (1, -1), (2, 1), (3, -1)], 6, 5),
    ([(0, 1), (1, -1)], [(0, 1), (1, -1), (2, 1), (3, -1)], 4, 7),
    ([(0, 1), (0, 1), (1, -1), (1, 1)], [(1, -1), (0, 1), (0, -1)], 3, 2),
])
def test_linear_matches_einsum(ins, outs, cin, cout):
    rng = np.random.default_rng(80)
    din = sum(2 * l + 1 for l, _ in ins)
    n = O.linear_num_weights(ins, outs)
    assert n == len(_pairs(ins, outs))
    x = rng.standard_normal((11, din, cin))
    W = rng.standard_normal((n, cin, cout))
    np.testing.assert_allclose(O.linear(ins, outs, x, W), _einsum_linear(ins, outs, x, W),
                               rtol=1e-13, atol=1e-13)


def test_linear_identity_and_unmatched_blocks():
    ins = [(0, 1), (1, -1), (2, 1)]
    outs = [(0, 1), (1, 1), (2, 1)]  # 1e has no source: stays zero
    rng = np.random.default_rng(81)
    x = rng.standard_normal((5, 9, 4))
    W = np.stack([np.eye(4)] * O.linear_num_weights(ins, outs))
    y = O.linear(ins, outs, x, W)
    np.testing.assert_array_equal(y[:, 0:1], x[:, 0:1])
    np.testing.assert_array_equal(y[:, 1:4], 0.0)
    np.testing.assert_array_equal(y[:, 4:9], x[:, 4:9])


def test_linear_sums_blocks_of_one_type():
    ins, outs = [(0, 1), (0, 1)], [(0, 1)]
    rng = np.random.default_rng(82)
    x = rng.standard_normal((3, 2, 2))
    W = rng.standard_normal((2, 2, 3))
    y = O.linear(ins, outs, x, W)
    np.testing.assert_allclose(y[:, 0], x[:, 0] @ W[0] + x[:, 1] @ W[1], rtol=1e-14)


def test_linear_rotation_equivariance():
    ins = outs = [(0, 1), (1, -1), (2, 1), (3, -1)]
    rng = np.random.default_rng(83)
    R = _rot(rng)
    x = rng.standard_normal((7, 16, 3))
    W = rng.standard_normal((4, 3, 5))
    y = O.linear(ins, outs, x, W)
    yr = O.linear(ins, outs, _block_rotate(ins, R, rng, x), W)
    np.testing.assert_allclose(yr, _block_rotate(outs, R, rng, y), atol=1e-11)


def test_linear_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.linear([(0, 1)], [(0, 1)], np.zeros((2, 1, 0)), np.zeros((1, 0, 1)))


def test_linear_backward_adjoint_and_finite_differences():
    # y is bilinear in (x, W): <dy, y> = <dx, x> = <dW, W>; and each
    # gradient entry equals a central difference of <dy, y>
    ins = [(0, 1), (1, -1), (0, 1), (2, 1)]
    outs = [(1, -1), (0, 1), (2, 1), (3, -1)]
    rng = np.random.default_rng(84)
    x = rng.standard_normal((6, _dim(ins), 3))
    W = rng.standard_normal((O.linear_num_weights(ins, outs), 3, 4))
    dy = rng.standard_normal((6, _dim(outs), 4))
    dx, dW = O.linear_backward(ins, outs, x, W, dy)
    ref = np.vdot(dy, O.linear(ins, outs, x, W))
    assert np.vdot(dx, x) == pytest.approx(ref, rel=1e-12)
    assert np.vdot(dW, W) == pytest.approx(ref, rel=1e-12)
    # the 3o output block has no source: its cotangent reaches nothing
    assert np.all(dx[:, :, :] == O.linear_backward(ins, outs, x, W, _zero_block(dy, outs, 3))[0])
    h = 1e-5
    loss = lambda x, W: np.vdot(dy, O.linear(ins, outs, x, W))
    for arr, grad, k in ((x, dx, 0), (W, dW, 1)):
        for _ in range(5):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p, args_m = [x, W], [x, W]
            args_p[k], args_m[k] = ap, am
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert fd == pytest.approx(grad[idx], rel=1e-7, abs=1e-9)


def test_linear_backward_matches_einsum():
    ins, outs = [(0, 1), (1, -1), (1, -1)], [(1, -1), (0, 1)]
    rng = np.random.default_rng(85)
    x = rng.standard_normal((9, 7, 4))
    W = rng.standard_normal((O.linear_num_weights(ins, outs), 4, 5))
    dy = rng.standard_normal((9, 4, 5))
    dx, dW = O.linear_backward(ins, outs, x, W, dy)
    io, oo = _offsets(ins), _offsets(outs)
    rdx, rdW = np.zeros_like(x), np.zeros_like(W)
    for n, (i, o) in enumerate(_pairs(ins, outs)):
        d = 2 * ins[i][0] + 1
        rdx[:, io[i]:io[i] + d] += np.einsum("rmc,kc->rmk", dy[:, oo[o]:oo[o] + d], W[n])
        rdW[n] = np.einsum("rmk,rmc->kc", x[:, io[i]:io[i] + d], dy[:, oo[o]:oo[o] + d])
    np.testing.assert_allclose(dx, rdx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW, rdW, rtol=1e-12, atol=1e-12)


def _dim(irreps):
    return sum(2 * l + 1 for l, _ in irreps)


def _zero_block(dy, outs, o):
    z = dy.copy()
    off = _offsets(outs)[o]
    z[:, off:off + 2 * outs[o][0] + 1] = 0.0
    return z
