"""GPU parity of the coefficient-table tensor product (e3_tp_forward_generic,
e3_tp_backward_generic)
through the C ABI, against the fp64 oracle, at the degrees of e3j's
tensor-product benchmarks (B.1 Figs 5-6: every irrep 0..L once, natural
parity for the symmetric paths, (-1)^(l+1) for the skew-symmetric ones,
C = 128).

Tolerance: max|gpu - oracle| / RMS(oracle) <= 1e-5 (fp32), 2e-2 ahead of the
output's own rounding for bf16 storage; against the compiled kernel on a
signature both serve, twice the fp32 gate (each side is within it).  y is
the harmonics of seeded random vectors (an input here), x and w N(0, 1).
"""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _irreps(L, skew=False):
    return [(l, (1 if l % 2 == 0 else -1) * (-1 if skew else 1)) for l in range(L + 1)]


def _case(L, C, B, seed, skew=False, per_path=False):
    from clebsch_gordan_tensor_amd import api
    xi = oi = _irreps(L, skew)
    yi = _irreps(L)
    flags = api.E3_OUT_PER_PATH if per_path else 0
    d = api.Desc(xi, yi, oi, C, flags)
    od = O.Desc(xi, yi, oi, C, per_path=per_path)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, d.dx, C)).astype(np.float32)
    y = O.sh(L, rng.standard_normal((B, 3))).astype(np.float32)
    w = rng.standard_normal((B, api.num_paths(d), C)).astype(np.float32)
    return d, od, x, y, w


@pytest.mark.parametrize("L,skew", [(1, False), (4, False), (5, False), (6, False), (6, True)])
def test_generic_tp_matches_oracle(gpu, L, skew):
    d, od, x, y, w = _case(L, 128, 97, 300 + L, skew)
    z = host(gpu.tp_forward_generic(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, f"generic tp L={L} skew={skew}")


@pytest.mark.parametrize("C", [1, 32, 97, 130, 192])
def test_generic_tp_channel_counts(gpu, C):
    d, od, x, y, w = _case(4, C, 41, 310 + C)
    z = host(gpu.tp_forward_generic(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, f"generic tp C={C}")


def test_generic_tp_per_path_outputs(gpu):
    d, od, x, y, w = _case(2, 64, 55, 320, per_path=True)
    assert d.dout == od.dout
    z = host(gpu.tp_forward_generic(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, "generic tp per path")


def test_generic_tp_bf16(gpu):
    from tests.gpu_util import S
    d, od, x, y, w = _case(4, 128, 77, 330)
    x, w = S.round_bf16(x), S.round_bf16(w)
    z = host(gpu.tp_forward_generic(d, dev(x, "bf16"), dev(y), dev(w, "bf16")))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_BF16, "generic tp bf16", bf16_out=True)


def test_generic_tp_equals_compiled_kernel(gpu):
    # a signature with a compiled kernel: 0e+1o+2e x harmonics 0..3 -> 0e+1o+2e+3o
    from clebsch_gordan_tensor_amd import api
    xi, yi, oi = _irreps(2), _irreps(3), _irreps(3)
    d = api.Desc(xi, yi, oi, 128)
    assert api.supported(d)
    rng = np.random.default_rng(340)
    B = 1000
    x = dev(rng.standard_normal((B, d.dx, 128)).astype(np.float32))
    y = dev(O.sh(3, rng.standard_normal((B, 3))).astype(np.float32))
    w = dev(rng.standard_normal((B, api.num_paths(d), 128)).astype(np.float32))
    a = gpu.tp_forward_generic(d, x, y, w)
    b = gpu.tp_forward(d, x, y, w)
    torch.cuda.synchronize()
    assert_close(host(a), host(b).astype(np.float64), 2 * TOL_F32, "generic vs compiled")


def test_generic_tp_full_size_sampled(gpu):
    # the benchmark's shape at L = 6: 32768 rows, 128 channels, 106 paths
    d, od, x, y, w = _case(6, 128, 32768, 350)
    z = gpu.tp_forward_generic(d, dev(x), dev(y), dev(w))
    z2 = gpu.tp_forward_generic(d, dev(x), dev(y), dev(w))
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int32), z2.view(torch.int32))
    rows = np.sort(np.random.default_rng(4).choice(32768, 60, replace=False))
    ref = O.tp_forward(od, x, y, w, rows=rows)
    assert_close(host(z)[rows], ref, TOL_F32, "generic tp L=6 sampled")


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("L,skew,C", [(2, False, 64), (4, False, 128), (6, False, 128),
                                      (5, True, 96)])
def test_generic_tp_backward_matches_oracle(gpu, L, skew, C):
    d, od, x, y, w = _case(L, C, 61, 360 + L, skew)
    dz = np.random.default_rng(361 + L).standard_normal((61, d.dout, C)).astype(np.float32)
    dx, dw, dy = gpu.tp_backward_generic(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    rdx, rdw, rdy = O.tp_backward(od, x, y, w, dz)
    for k, a, b in (("dx", dx, rdx), ("dw", dw, rdw), ("dy", dy, rdy)):
        assert_close(host(a), b, TOL_F32, f"generic tp backward L={L} skew={skew}:{k}")


def test_generic_tp_backward_per_path_and_bf16(gpu):
    from tests.gpu_util import S
    d, od, x, y, w = _case(2, 64, 40, 370, per_path=True)
    dz = np.random.default_rng(371).standard_normal((40, d.dout, 64)).astype(np.float32)
    got = gpu.tp_backward_generic(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    for k, a, b in zip(("dx", "dw", "dy"), got, O.tp_backward(od, x, y, w, dz)):
        assert_close(host(a), b, TOL_F32, f"generic tp backward per path:{k}")
    d, od, x, y, w = _case(4, 128, 50, 372)
    dz = np.random.default_rng(373).standard_normal((50, d.dout, 128)).astype(np.float32)
    x, w, dz = S.round_bf16(x), S.round_bf16(w), S.round_bf16(dz)
    got = gpu.tp_backward_generic(d, dev(x, "bf16"), dev(y), dev(w, "bf16"), dev(dz, "bf16"))
    torch.cuda.synchronize()
    for k, a, b in zip(("dx", "dw", "dy"), got, O.tp_backward(od, x, y, w, dz)):
        assert_close(host(a), b, TOL_BF16, f"generic tp backward bf16:{k}", bf16_out=k != "dy")


def test_generic_tp_backward_equals_compiled_kernel(gpu):
    from clebsch_gordan_tensor_amd import api
    xi, yi, oi = _irreps(2), _irreps(3), _irreps(3)
    d = api.Desc(xi, yi, oi, 128)
    rng = np.random.default_rng(380)
    B = 700
    x = dev(rng.standard_normal((B, d.dx, 128)).astype(np.float32))
    y = dev(O.sh(3, rng.standard_normal((B, 3))).astype(np.float32))
    w = dev(rng.standard_normal((B, api.num_paths(d), 128)).astype(np.float32))
    dz = dev(rng.standard_normal((B, d.dout, 128)).astype(np.float32))
    a = gpu.tp_backward_generic(d, x, y, w, dz)
    b = gpu.tp_backward(d, x, y, w, dz)
    torch.cuda.synchronize()
    for k, u, v in zip(("dx", "dw", "dy"), a, b):
        assert_close(host(u), host(v).astype(np.float64), 2 * TOL_F32, f"generic vs compiled:{k}")


# ---------------------------------------------------- harmonics up to degree 8

@pytest.mark.parametrize("lmax", [6, 7, 8])
def test_harmonics_to_high_degree_match_oracle(gpu, lmax):
    # the library builds degrees 4..8 by coupling Y_1 with Y_{L-1} (Gaunt
    # relation); the oracle by the Legendre construction
    rng = np.random.default_rng(390)
    v = (rng.standard_normal((5001, 3)) * rng.uniform(0.1, 10, (5001, 1))).astype(np.float32)
    v[7] = 0.0
    v[8] = [0.0, 0.0, 3.0]
    Y = host(gpu.spherical_harmonics(lmax, dev(v)))
    ref = O.sh(lmax, v)
    for l in range(lmax + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        assert_close(Y[:, sl], ref[:, sl], TOL_F32, f"harmonics l={l}")
    assert np.all(Y[7, 1:] == 0.0) and Y[7, 0] == 1.0


@pytest.mark.parametrize("lmax", [4, 6, 7, 8])
def test_harmonics_gradient_to_high_degree(gpu, lmax):
    # the vector gradient through the coupling recursion, against the
    # fourth-order differences of the oracle's harmonics
    rng = np.random.default_rng(391 + lmax)
    v = (rng.standard_normal((3001, 3)) * rng.uniform(0.1, 10, (3001, 1))).astype(np.float32)
    v[5] = 0.0
    dY = rng.standard_normal((3001, (lmax + 1) ** 2)).astype(np.float32)
    g = host(gpu.spherical_harmonics_backward(lmax, dev(v), dev(dY)))
    assert_close(g, O.sh_grad_fd(lmax, v, dY), TOL_F32, f"harmonics gradient l<={lmax}")
    assert np.all(g[5] == 0.0)


@pytest.mark.parametrize("C", [97, 130])
def test_generic_tp_backward_odd_channel_counts(gpu, C):
    # two channels per lane with an odd count or a partial second chunk
    d, od, x, y, w = _case(3, C, 45, 395 + C)
    dz = np.random.default_rng(396).standard_normal((45, d.dout, C)).astype(np.float32)
    got = gpu.tp_backward_generic(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    for k, a, b in zip(("dx", "dw", "dy"), got, O.tp_backward(od, x, y, w, dz)):
        assert_close(host(a), b, TOL_F32, f"generic tp backward C={C}:{k}")
