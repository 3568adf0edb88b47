"""GPU parity of the coefficient-table convolution (e3_conv_forward_generic,
e3_conv_backward_generic) through the C ABI, against the fp64 oracle, at the
degrees of e3j's higher-degree convolution benchmark (B.1 Fig 7: every
irrep 0..L once, SH l <= L, 128 channels, 2,048 nodes with about 45
neighbours).

Tolerance: max|gpu - oracle| / RMS(oracle) <= 1e-5 (fp32), 2e-2 ahead of the
output's own rounding for bf16 storage; against the compiled kernels on a
signature both serve, twice the fp32 gate (each side is within it).  Small
graphs compare every element; the full-size graph compares sampled rows.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_close, dev, edges_of_receivers,
                            edges_of_senders, host, subgraph)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _problem(xi, yi, oi, C, n, box, rc, seed, pad=0, dtype="f32"):
    rng = np.random.default_rng(seed)
    g = S.random_graph(n, box, rc, seed)
    if pad:
        from tests.test_oracle_conv import with_padding
        g = with_padding(g, pad, seed)
    P = S.num_paths(xi, yi, oi)
    x = rng.standard_normal((n, S.dim(xi), C)).astype(np.float32)
    w = rng.standard_normal((g.n_edges, P, C)).astype(np.float32)
    dm = rng.standard_normal((n, S.dim(oi), C)).astype(np.float32)
    if dtype == "bf16":
        x, w, dm = S.round_bf16(x), S.round_bf16(w), S.round_bf16(dm)
    return g, x, w, dm


def _run(gpu, d, g, x, w, dm, dtype="f32", Y=None):
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    ysrc = dev(Y.astype(np.float32)) if Y is not None else dev(g.evec)
    xd, wd, dmd = dev(x, dtype), dev(w, dtype), dev(dm, dtype)
    ws = gpu.conv_prepare_transpose(rowptr, sender, edge_vec=None if Y is not None else ysrc)
    m = gpu.conv_forward_generic(d, rowptr, sender, ysrc, xd, wd, workspace=ws)
    m0 = gpu.conv_forward_generic(d, rowptr, sender, ysrc, xd, wd)
    dx, dw, dY = gpu.conv_backward_generic(d, rowptr, sender, ws, ysrc, xd, wd, dmd)
    dx2, dw2, dY2 = gpu.conv_backward_generic(d, rowptr, sender, ws, ysrc, xd, wd, dmd)
    torch.cuda.synchronize()
    # the node order changes only which wavefront takes a node; reruns repeat
    for a, b in ((m, m0), (dx, dx2), (dw, dw2), (dY, dY2)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
    return host(m), host(dx), host(dw), host(dY)


def _oracle(od, g, x, w, dm, Y=None):
    kw = dict(Y=Y) if Y is not None else dict(evec=g.evec)
    m = O.conv_forward(od, g.rowptr, g.sender, x, w, **kw)
    dx = O.conv_backward_dx(od, g.rowptr, g.sender, w, dm, **kw)
    dw, dY = O.conv_backward_edge(od, g.rowptr, g.sender, x, w, dm, **kw)
    return m, dx, dw, dY


def _check(got, ref, tol, name):
    bf = tol == TOL_BF16
    for k, a, b in zip(("m", "dx", "dw", "dY"), got, ref):
        assert_close(a, b, tol, f"{name}:{k}", bf16_out=bf and k != "dY")


@pytest.mark.parametrize("L,skew,C", [(1, False, 32), (2, False, 128), (3, False, 97),
                                      (4, False, 96), (6, False, 128), (5, True, 64)])
def test_generic_conv_matches_oracle(gpu, L, skew, C):
    xi = oi = S.degree_irreps(L, skew)
    yi = S.sh_irreps(L)
    n = 40 if L >= 5 else 64
    g, x, w, dm = _problem(xi, yi, oi, C, n, 7.0, 3.5, seed=400 + L)
    d = gpu.Desc(xi, yi, oi, C)
    got = _run(gpu, d, g, x, w, dm)
    ref = _oracle(O.Desc(xi, yi, oi, C), g, x, w, dm)
    _check(got, ref, TOL_F32, f"generic conv L={L} skew={skew} C={C}")


def test_generic_conv_given_harmonics_and_padding(gpu):
    # Y given (arbitrary rows, not harmonics), padding edges in every segment
    xi = oi = S.degree_irreps(4)
    yi = S.sh_irreps(4)
    g, x, w, dm = _problem(xi, yi, oi, 64, 50, 7.0, 3.5, seed=410, pad=2)
    Y = np.random.default_rng(411).standard_normal((g.n_edges, S.dim(yi))).astype(np.float32)
    d = gpu.Desc(xi, yi, oi, 64, gpu.E3_Y_GIVEN)
    got = _run(gpu, d, g, x, w, dm, Y=Y)
    ref = _oracle(O.Desc(xi, yi, oi, 64), g, x, w, dm, Y=Y)
    _check(got, ref, TOL_F32, "generic conv Y given + padding")
    pad = g.sender < 0
    assert np.all(got[2][pad] == 0) and np.all(got[3][pad] == 0)


def test_generic_conv_padding_from_vectors(gpu):
    xi = oi = S.degree_irreps(3)
    yi = S.sh_irreps(3)
    g, x, w, dm = _problem(xi, yi, oi, 32, 50, 7.0, 3.5, seed=412, pad=1)
    d = gpu.Desc(xi, yi, oi, 32)
    got = _run(gpu, d, g, x, w, dm)
    ref = _oracle(O.Desc(xi, yi, oi, 32), g, x, w, dm)
    _check(got, ref, TOL_F32, "generic conv padding")


def test_generic_conv_harmonics_subset(gpu):
    # y = 1o + 3o only (edge-vector mode picks those degrees' harmonics)
    xi = S.degree_irreps(2)
    yi = [(1, -1), (3, -1)]
    oi = [(1, -1), (2, 1), (3, -1), (4, 1)]
    g, x, w, dm = _problem(xi, yi, oi, 64, 60, 7.0, 3.5, seed=413)
    d = gpu.Desc(xi, yi, oi, 64)
    got = _run(gpu, d, g, x, w, dm)
    ref = _oracle(O.Desc(xi, yi, oi, 64), g, x, w, dm)
    _check(got, ref, TOL_F32, "generic conv y subset")


def test_generic_conv_per_path_and_bf16(gpu):
    xi = oi = S.degree_irreps(2)
    yi = S.sh_irreps(2)
    g, x, w, dm0 = _problem(xi, yi, oi, 64, 50, 7.0, 3.5, seed=414)
    d = gpu.Desc(xi, yi, oi, 64, gpu.E3_OUT_PER_PATH)
    od = O.Desc(xi, yi, oi, 64, per_path=True)
    dm = np.random.default_rng(415).standard_normal((50, od.dout, 64)).astype(np.float32)
    got = _run(gpu, d, g, x, w, dm)
    _check(got, _oracle(od, g, x, w, dm), TOL_F32, "generic conv per path")
    xi = oi = S.degree_irreps(4)
    yi = S.sh_irreps(4)
    g, x, w, dm = _problem(xi, yi, oi, 128, 50, 7.0, 3.5, seed=416, dtype="bf16")
    d = gpu.Desc(xi, yi, oi, 128)
    got = _run(gpu, d, g, x, w, dm, dtype="bf16")
    _check(got, _oracle(O.Desc(xi, yi, oi, 128), g, x, w, dm), TOL_BF16, "generic conv bf16")


def test_generic_conv_equals_compiled_kernels(gpu):
    xi, yi, oi = S.parse_irreps("0e+1o")[1], S.sh_irreps(3), S.parse_irreps("0e+1o+2e+3o")[1]
    g, x, w, dm = _problem(xi, yi, oi, 128, 300, 12.0, 4.0, seed=417)
    d = gpu.Desc(xi, yi, oi, 128)
    assert gpu.supported(d)
    a = _run(gpu, d, g, x, w, dm)
    rowptr, sender, ev = dev(g.rowptr), dev(g.sender), dev(g.evec)
    xd, wd, dmd = dev(x), dev(w), dev(dm)
    ws = gpu.conv_prepare_transpose(rowptr, sender, edge_vec=ev)
    b = (gpu.conv_forward(d, rowptr, sender, ev, xd, wd, workspace=ws),
         *gpu.conv_backward(d, rowptr, sender, ws, ev, xd, wd, dmd))
    torch.cuda.synchronize()
    for k, u, v in zip(("m", "dx", "dw", "dY"), a, b):
        assert_close(u, host(v).astype(np.float64), 2 * TOL_F32, f"generic vs compiled:{k}")


def test_generic_conv_isolated_and_empty_nodes(gpu):
    # nodes far apart: no edges at all for most receivers -> m = 0, dx = 0
    xi = oi = S.degree_irreps(2)
    yi = S.sh_irreps(2)
    g, x, w, dm = _problem(xi, yi, oi, 32, 30, 60.0, 6.0, seed=418)
    assert (np.diff(g.rowptr) == 0).any()
    d = gpu.Desc(xi, yi, oi, 32)
    got = _run(gpu, d, g, x, w, dm)
    _check(got, _oracle(O.Desc(xi, yi, oi, 32), g, x, w, dm), TOL_F32, "generic conv sparse")
    lonely = np.diff(g.rowptr) == 0
    assert np.all(got[0][lonely] == 0)


def test_generic_conv_full_size_sampled(gpu):
    # the higher-degree benchmark graph at L = 6: 2,048 nodes, ~45 neighbours
    p = S.make_conv_degree(6)
    g = p.graph
    d = gpu.Desc(p.x_irreps, p.y_irreps, p.out_irreps, p.channels)
    od = O.Desc(p.x_irreps, p.y_irreps, p.out_irreps, p.channels)
    m, dx, dw, dY = _run(gpu, d, g, p.x, p.w, p.dm)
    rng = np.random.default_rng(419)
    nodes = np.sort(rng.choice(g.n_nodes, 12, replace=False))
    edges = np.sort(rng.choice(g.n_edges, 24, replace=False))
    rp, sn, ev, ids = edges_of_receivers(g, nodes)
    assert_close(m[nodes], O.conv_forward(od, rp, sn, p.x, p.w[ids], evec=ev, rows=nodes),
                 TOL_F32, "deg6:m")
    rp, sn, ev, ids = edges_of_senders(g, nodes)
    assert_close(dx[nodes], O.conv_backward_dx(od, rp, sn, p.w[ids], p.dm, evec=ev, rows=nodes),
                 TOL_F32, "deg6:dx")
    rp, sn, ev, ids = subgraph(g, edges)
    rdw, rdY = O.conv_backward_edge(od, rp, sn, p.x, p.w[ids], p.dm, evec=ev)
    assert_close(dw[edges], rdw, TOL_F32, "deg6:dw")
    assert_close(dY[edges], rdY, TOL_F32, "deg6:dY")


def test_generic_conv_graph_without_edges(gpu):
    # nodes but no edges: m = 0 and dx = 0, empty edge cotangents
    xi = oi = S.degree_irreps(3)
    yi = S.sh_irreps(3)
    n, C = 20, 64
    d = gpu.Desc(xi, yi, oi, C)
    rowptr = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    sender = torch.zeros(0, dtype=torch.int32, device="cuda")
    ev = torch.zeros((0, 3), device="cuda")
    x = dev(np.random.default_rng(420).standard_normal((n, S.dim(xi), C)).astype(np.float32))
    w = torch.zeros((0, S.num_paths(xi, yi, oi), C), device="cuda")
    dm = dev(np.random.default_rng(421).standard_normal((n, S.dim(oi), C)).astype(np.float32))
    ws = gpu.conv_prepare_transpose(rowptr, sender)
    m = gpu.conv_forward_generic(d, rowptr, sender, ev, x, w, workspace=ws)
    dx, dw, dY = gpu.conv_backward_generic(d, rowptr, sender, ws, ev, x, w, dm)
    torch.cuda.synchronize()
    assert torch.count_nonzero(m) == 0 and torch.count_nonzero(dx) == 0
    assert dw.numel() == 0 and dY.numel() == 0


def test_generic_tables_at_degrees_7_and_8(gpu):
    # the coefficient tables past degree 6, on operands within their 63
    # components: x 8e, harmonics 0e+2e+8e and 7o given (rows of any values),
    # out 8e+6e+7o; the convolution forward and backward and the tensor
    # product forward and backward
    xi, oi = [(8, 1)], [(8, 1), (6, 1), (7, -1)]
    yi = [(0, 1), (2, 1), (8, 1), (7, -1)]
    g, x, w, dm = _problem(xi, yi, oi, 64, 40, 7.0, 3.5, seed=430, pad=1)
    Y = np.random.default_rng(431).standard_normal((g.n_edges, S.dim(yi))).astype(np.float32)
    d = gpu.Desc(xi, yi, oi, 64, gpu.E3_Y_GIVEN)
    od = O.Desc(xi, yi, oi, 64)
    got = _run(gpu, d, g, x, w, dm, Y=Y)
    _check(got, _oracle(od, g, x, w, dm, Y=Y), TOL_F32, "generic conv degree 8")
    rng = np.random.default_rng(432)
    B = 53
    xt = rng.standard_normal((B, S.dim(xi), 64)).astype(np.float32)
    yt = rng.standard_normal((B, S.dim(yi))).astype(np.float32)
    wt = rng.standard_normal((B, S.num_paths(xi, yi, oi), 64)).astype(np.float32)
    dz = rng.standard_normal((B, S.dim(oi), 64)).astype(np.float32)
    z = host(gpu.tp_forward_generic(d, dev(xt), dev(yt), dev(wt)))
    assert_close(z, O.tp_forward(od, xt, yt, wt), TOL_F32, "generic tp degree 8")
    dx, dw, dy = gpu.tp_backward_generic(d, dev(xt), dev(yt), dev(wt), dev(dz))
    for k, a, b in zip(("dx", "dw", "dy"), (dx, dw, dy), O.tp_backward(od, xt, yt, wt, dz)):
        assert_close(host(a), b, TOL_F32, f"generic tp bwd degree 8:{k}")
