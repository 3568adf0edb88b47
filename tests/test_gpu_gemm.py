"""GPU parity of the tensor product as dense products on the fp32 matrix
cores (e3_tp_forward_gemm) through the C ABI, against the fp64 oracle, at the
degrees of e3j's tensor-product benchmarks (B.1 Figs 5-6: every irrep 0..L
once, natural or skew-symmetric parities, C = 128), per-path outputs, channel
counts that take 16-, 64- and 128-channel slabs, and the benchmark's 32,768
rows at L = 6 on sampled rows.

Tolerance: max|gpu - oracle| / RMS(oracle) <= 1e-5 (fp32); against the
coefficient-table kernel on the same inputs, twice that (each is within it).
y is the harmonics of seeded random vectors (an input here), x and w N(0, 1).
"""
import numpy as np
import pytest

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


@pytest.mark.parametrize("L,skew", [(1, False), (2, False), (3, False), (4, False), (5, False),
                                    (6, False), (6, True), (7, False), (7, True), (8, False),
                                    (8, True)])
def test_gemm_tp_matches_oracle(gpu, L, skew):
    d, od, x, y, w = _case(L, 128, 97, 500 + L, skew)
    z = host(gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, f"gemm tp L={L} skew={skew}")


@pytest.mark.parametrize("C", [16, 48, 64, 256])
def test_gemm_tp_channels(gpu, C):
    d, od, x, y, w = _case(4, C, 37, 520 + C)
    z = host(gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, f"gemm tp C={C}")


def test_gemm_tp_per_path_outputs(gpu):
    d, od, x, y, w = _case(3, 64, 41, 540, per_path=True)
    assert d.dout == od.dout
    z = host(gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w)))
    assert_close(z, O.tp_forward(od, x, y, w), TOL_F32, "gemm tp per path")


def test_gemm_tp_equals_table_kernel(gpu):
    d, od, x, y, w = _case(5, 128, 300, 550)
    a = gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w))
    b = gpu.tp_forward_generic(d, dev(x), dev(y), dev(w))
    torch.cuda.synchronize()
    assert_close(host(a), host(b).astype(np.float64), 2 * TOL_F32, "gemm vs table kernel")


def test_gemm_tp_rejects_unsupported(gpu):
    from clebsch_gordan_tensor_amd import api
    d, od, x, y, w = _case(2, 24, 3, 560)  # C % 16 != 0
    with pytest.raises(api.E3Error):
        gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w))


def test_gemm_tp_full_size_sampled(gpu):
    # the benchmark's shape at L = 6: 32768 rows, 128 channels, 106 paths
    d, od, x, y, w = _case(6, 128, 32768, 570)
    z = gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w))
    z2 = gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w))
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int32), z2.view(torch.int32))
    rows = np.sort(np.random.default_rng(5).choice(32768, 60, replace=False))
    ref = O.tp_forward(od, x, y, w, rows=rows)
    assert_close(host(z)[rows], ref, TOL_F32, "gemm tp L=6 sampled")


# --------------------------------------------------------- convolution

def _conv_problem(L, C, n, seed, pad=0, skew=False):
    from clebsch_gordan_tensor_amd import api
    from clebsch_gordan_tensor_amd import synth as S
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
    Y = O.sh(L, g.evec.astype(np.float64)).astype(np.float32)
    return d, od, g, x, w, Y


@pytest.mark.parametrize("L,C,skew", [(1, 64, False), (3, 128, False), (4, 64, False),
                                      (6, 128, False), (6, 48, True), (7, 128, False),
                                      (7, 32, True), (8, 128, False), (8, 32, True)])
def test_gemm_conv_matches_oracle(gpu, L, C, skew):
    d, od, g, x, w, Y = _conv_problem(L, C, 40 if L >= 5 else 64, 600 + L, skew=skew)
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    m = gpu.conv_forward_gemm(d, rowptr, sender, dev(Y), dev(x), dev(w))
    m2 = gpu.conv_forward_gemm(d, rowptr, sender, dev(Y), dev(x), dev(w))
    torch.cuda.synchronize()
    assert torch.equal(m.view(torch.int32), m2.view(torch.int32))
    ref = O.conv_forward(od, g.rowptr, g.sender, x, w, Y=Y)
    assert_close(host(m), ref, TOL_F32, f"gemm conv L={L} C={C}")


def test_gemm_conv_padding_and_empty_rows(gpu):
    # padding edges (sender < 0) add nothing; receivers without edges get 0
    d, od, g, x, w, Y = _conv_problem(3, 64, 50, 620, pad=7)
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    m = host(gpu.conv_forward_gemm(d, rowptr, sender, dev(Y), dev(x), dev(w)))
    ref = O.conv_forward(od, g.rowptr, g.sender, x, w, Y=Y)
    assert_close(m, ref, TOL_F32, "gemm conv padding")
    empty = np.flatnonzero(np.diff(g.rowptr) == 0)
    assert np.all(m[empty] == 0)


def test_gemm_conv_equals_table_kernel(gpu):
    d, od, g, x, w, Y = _conv_problem(5, 128, 60, 630)
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    a = gpu.conv_forward_gemm(d, rowptr, sender, dev(Y), dev(x), dev(w))
    b = gpu.conv_forward_generic(d, rowptr, sender, dev(Y), dev(x), dev(w))
    torch.cuda.synchronize()
    assert_close(host(a), host(b).astype(np.float64), 2 * TOL_F32, "gemm conv vs table kernel")


@pytest.mark.parametrize("L", [2, 6, 7])
def test_gemm_conv_from_edge_vectors(gpu, L):
    # the harmonics computed per edge from the vectors, against the oracle
    from clebsch_gordan_tensor_amd import api
    d, od, g, x, w, Y = _conv_problem(L, 64, 40, 640 + L)
    dv = api.Desc(d.x, d.y, d.out, 64)
    m = host(gpu.conv_forward_gemm(dv, dev(g.rowptr), dev(g.sender), dev(g.evec), dev(x), dev(w)))
    ref = O.conv_forward(od, g.rowptr, g.sender, x, w, evec=g.evec)
    assert_close(m, ref, TOL_F32, f"gemm conv from vectors L={L}")


def test_gemm_pathless_output_block(gpu):
    # 0o is reached by no path of 0e+1o (x) 0e+1o: its rows are zero and the
    # blocks that paths do reach keep their own values (the plan gives every
    # output block its own rows)
    from clebsch_gordan_tensor_amd import api
    from clebsch_gordan_tensor_amd import synth as S
    xi, yi, oi = [(0, 1), (1, -1)], [(0, 1), (1, -1)], [(0, 1), (1, -1), (0, -1)]
    C, B = 16, 33
    d, od = api.Desc(xi, yi, oi, C), O.Desc(xi, yi, oi, C)
    rng = np.random.default_rng(575)
    x = rng.standard_normal((B, 4, C)).astype(np.float32)
    y = O.sh(1, rng.standard_normal((B, 3))).astype(np.float32)
    w = rng.standard_normal((B, api.num_paths(d), C)).astype(np.float32)
    ref = O.tp_forward(od, x, y, w)
    assert np.all(ref[:, 4] == 0) and np.abs(ref[:, 0]).max() > 0
    z = host(gpu.tp_forward_gemm(d, dev(x), dev(y), dev(w)))
    assert_close(z, ref, TOL_F32, "gemm tp with a pathless block")
    assert np.all(z[:, 4] == 0)
    g = S.random_graph(48, 6.0, 3.0, 576)
    dg = api.Desc(xi, yi, oi, C, api.E3_Y_GIVEN)
    xn = rng.standard_normal((48, 4, C)).astype(np.float32)
    wn = rng.standard_normal((g.n_edges, api.num_paths(d), C)).astype(np.float32)
    Y = O.sh(1, g.evec.astype(np.float64)).astype(np.float32)
    m = host(gpu.conv_forward_gemm(dg, dev(g.rowptr), dev(g.sender), dev(Y), dev(xn), dev(wn)))
    ref = O.conv_forward(od, g.rowptr, g.sender, xn, wn, Y=Y)
    assert_close(m, ref, TOL_F32, "gemm conv with a pathless block")
    assert np.all(m[:, 4] == 0)


def test_gemm_conv_sender_out_of_range_is_padding(gpu):
    # any sender outside [0, N) marks a padding edge: sender = N adds nothing
    d, od, g, x, w, Y = _conv_problem(3, 64, 50, 650)
    snd = g.sender.copy()
    hit = np.random.default_rng(651).choice(g.n_edges, 9, replace=False)
    snd[hit] = g.n_nodes
    snd[hit[:3]] = g.n_nodes + 1000
    m = host(gpu.conv_forward_gemm(d, dev(g.rowptr), dev(snd), dev(Y), dev(x), dev(w)))
    ref_snd = snd.copy()
    ref_snd[hit] = -1
    ref = O.conv_forward(od, g.rowptr, ref_snd, x, w, Y=Y)
    assert_close(m, ref, TOL_F32, "gemm conv, senders past N")
