"""GPU parity of the dense-product backward (e3_tp_backward_gemm,
e3_conv_backward_gemm: dx, dw and dy as products on the fp32 matrix cores)
through the C ABI, against the fp64 oracle, at the degrees of e3j's
benchmarks (B.1 Figs 5-7: every irrep 0..L once, natural and skew parities),
per-path outputs, channel counts that take different slabs, an output irrep
no path reaches, padding edges and receivers without edges; and against the
coefficient-table backward on the same inputs.

Tolerance: max|gpu - oracle| / RMS(oracle) <= 1e-5 per output (fp32); against
the table kernel, twice that (each is within it).  y (or Y) is the harmonics
of seeded random vectors, x, w and the cotangent N(0, 1)."""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from tests.gpu_util import TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _tp_case(L, C, B, seed, skew=False, per_path=False, out=None):
    from clebsch_gordan_tensor_amd import api
    xi = S.degree_irreps(L, skew)
    oi = out if out is not None else xi
    yi = S.sh_irreps(L)
    d = api.Desc(xi, yi, oi, C, api.E3_OUT_PER_PATH if per_path else 0)
    od = O.Desc(xi, yi, oi, C, per_path=per_path)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, d.dx, C)).astype(np.float32)
    y = O.sh(L, rng.standard_normal((B, 3))).astype(np.float32)
    w = rng.standard_normal((B, api.num_paths(d), C)).astype(np.float32)
    dz = rng.standard_normal((B, d.dout, C)).astype(np.float32)
    return d, od, x, y, w, dz


def _check_tp(gpu, d, od, x, y, w, dz, what):
    got = gpu.tp_backward_gemm(d, dev(x), dev(y), dev(w), dev(dz))
    again = gpu.tp_backward_gemm(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for k, a, b in zip(("dx", "dw", "dy"), got, O.tp_backward(od, x, y, w, dz)):
        assert_close(host(a), b, TOL_F32, f"{what}:{k}")
    return got


@pytest.mark.parametrize("L,skew", [(1, False), (2, False), (3, False), (4, False), (5, False),
                                    (6, False), (6, True), (7, False), (7, True), (8, False),
                                    (8, True)])
def test_gemm_tp_backward_matches_oracle(gpu, L, skew):
    _check_tp(gpu, *_tp_case(L, 128, 61, 700 + L, skew), f"gemm tp bwd L={L} skew={skew}")


@pytest.mark.parametrize("C", [16, 48, 256])
def test_gemm_tp_backward_channels(gpu, C):
    _check_tp(gpu, *_tp_case(4, C, 23, 720 + C), f"gemm tp bwd C={C}")


def test_gemm_tp_backward_per_path_and_pathless(gpu):
    _check_tp(gpu, *_tp_case(3, 64, 29, 740, per_path=True), "gemm tp bwd per path")
    _check_tp(gpu, *_tp_case(1, 16, 31, 741, out=[(0, 1), (1, -1), (0, -1)]),
              "gemm tp bwd pathless block")


def test_gemm_tp_backward_equals_table_kernel(gpu):
    d, od, x, y, w, dz = _tp_case(5, 128, 200, 750)
    a = gpu.tp_backward_gemm(d, dev(x), dev(y), dev(w), dev(dz))
    b = gpu.tp_backward_generic(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    for k, u, v in zip(("dx", "dw", "dy"), a, b):
        assert_close(host(u), host(v).astype(np.float64), 2 * TOL_F32, f"gemm vs table:{k}")


def test_gemm_tp_backward_full_size_sampled(gpu):
    # the benchmark's shape at L = 6: 32768 rows, 128 channels, 106 paths
    d, od, x, y, w, dz = _tp_case(6, 128, 32768, 760)
    got = gpu.tp_backward_gemm(d, dev(x), dev(y), dev(w), dev(dz))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(32768, 40, replace=False))
    for k, a, b in zip(("dx", "dw", "dy"), got, O.tp_backward(od, x, y, w, dz, rows=rows)):
        assert_close(host(a)[rows], b, TOL_F32, f"gemm tp bwd L=6 sampled:{k}")


# --------------------------------------------------------- convolution

def _conv_case(L, C, n, seed, pad=0, skew=False):
    from clebsch_gordan_tensor_amd import api
    xi = oi = S.degree_irreps(L, skew)
    yi = S.sh_irreps(L)
    rng = np.random.default_rng(seed)
    g = S.random_graph(n, 7.0, 3.5, seed)
    if pad:
        from tests.test_oracle_conv import with_padding
        g = with_padding(g, pad, seed)
    d = api.Desc(xi, yi, oi, C, api.E3_Y_GIVEN)
    od = O.Desc(xi, yi, oi, C)
    P = api.num_paths(d)
    x = rng.standard_normal((n, d.dx, C)).astype(np.float32)
    w = rng.standard_normal((g.n_edges, P, C)).astype(np.float32)
    dm = rng.standard_normal((n, d.dout, C)).astype(np.float32)
    Y = O.sh(L, g.evec.astype(np.float64)).astype(np.float32)
    return d, od, g, x, w, dm, Y


def _run_conv(gpu, d, g, x, w, dm, Y):
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    ws = gpu.conv_prepare_transpose(rowptr, sender)
    got = gpu.conv_backward_gemm(d, rowptr, sender, ws, dev(Y), dev(x), dev(w), dev(dm))
    again = gpu.conv_backward_gemm(d, rowptr, sender, ws, dev(Y), dev(x), dev(w), dev(dm))
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    return [host(a) for a in got]


def _conv_ref(od, g, x, w, dm, Y):
    dx = O.conv_backward_dx(od, g.rowptr, g.sender, w, dm, Y=Y)
    dw, dY = O.conv_backward_edge(od, g.rowptr, g.sender, x, w, dm, Y=Y)
    return dx, dw, dY


@pytest.mark.parametrize("L,C,skew", [(1, 64, False), (3, 128, False), (4, 64, False),
                                      (6, 128, False), (6, 48, True), (7, 128, False),
                                      (7, 32, True), (8, 128, False), (8, 32, True)])
def test_gemm_conv_backward_matches_oracle(gpu, L, C, skew):
    d, od, g, x, w, dm, Y = _conv_case(L, C, 40 if L >= 5 else 64, 800 + L, skew=skew)
    got = _run_conv(gpu, d, g, x, w, dm, Y)
    for k, a, b in zip(("dx", "dw", "dY"), got, _conv_ref(od, g, x, w, dm, Y)):
        assert_close(a, b, TOL_F32, f"gemm conv bwd L={L} C={C}:{k}")


def test_gemm_conv_backward_padding_and_empty_rows(gpu):
    d, od, g, x, w, dm, Y = _conv_case(3, 64, 50, 820, pad=7)
    got = _run_conv(gpu, d, g, x, w, dm, Y)
    for k, a, b in zip(("dx", "dw", "dY"), got, _conv_ref(od, g, x, w, dm, Y)):
        assert_close(a, b, TOL_F32, f"gemm conv bwd padding:{k}")
    pad = g.sender < 0
    assert np.all(got[1][pad] == 0) and np.all(got[2][pad] == 0)
    lonely = np.setdiff1d(np.arange(g.n_nodes), g.sender[g.sender >= 0])
    assert np.all(got[0][lonely] == 0)


def test_gemm_conv_backward_equals_table_kernel(gpu):
    d, od, g, x, w, dm, Y = _conv_case(5, 128, 60, 830)
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    ws = gpu.conv_prepare_transpose(rowptr, sender)
    a = gpu.conv_backward_gemm(d, rowptr, sender, ws, dev(Y), dev(x), dev(w), dev(dm))
    b = gpu.conv_backward_generic(d, rowptr, sender, ws, dev(Y), dev(x), dev(w), dev(dm))
    torch.cuda.synchronize()
    for k, u, v in zip(("dx", "dw", "dY"), a, b):
        assert_close(host(u), host(v).astype(np.float64), 2 * TOL_F32, f"gemm conv vs table:{k}")


def test_gemm_conv_backward_needs_given_harmonics(gpu):
    from clebsch_gordan_tensor_amd import api
    d, od, g, x, w, dm, Y = _conv_case(2, 16, 20, 840)
    dv = api.Desc(d.x, d.y, d.out, 16)
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    ws = gpu.conv_prepare_transpose(rowptr, sender)
    with pytest.raises(api.E3Error) as ei:
        gpu.conv_backward_gemm(dv, rowptr, sender, ws, dev(Y), dev(x), dev(w), dev(dm))
    assert ei.value.status == -3
