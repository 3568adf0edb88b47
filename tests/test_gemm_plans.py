"""CPU checks of the dense-product plans the library builds on the host
(tables E3_GEN_GEMM, E3_GEN_GEMM_DX, E3_GEN_GEMM_DW, E3_GEN_GEMM_DY): a numpy
reading of each plan, doing what the matrix-core kernels do with it (A built
per row from y, one product per block over its K list), against the fp64
oracle's tensor product and its backward, at degrees 1-8 with natural and
skew parities, collapsed and per-path outputs, and an output irrep no path
reaches.  These pin the host logic; the GPU tests pin the kernels."""
import ctypes as C

import numpy as np
import pytest

from clebsch_gordan_tensor_amd import api
from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O

HDR = 16


def _plan(d, table):
    L = api.lib()
    n = C.c_size_t()
    assert L.e3_generic_plan_size(C.byref(d.c()), table, C.byref(n)) == 0, L.e3_last_error()
    buf = np.zeros(n.value // 4, np.int32)
    assert L.e3_generic_plan_build(C.byref(d.c()), table, buf.ctypes.data, n.value) == 0
    return buf


def _A(plan, y):
    """A (all blocks) for each row: A[at] = c1 y[y1] + c2 y[y2]."""
    a_floats, off_groups, n_groups = plan[9], plan[12], plan[7]
    g = plan[off_groups:off_groups + 4 * n_groups].reshape(-1, 4)
    # entries sorted by A index: the kernels' windows of A each take one run
    assert np.all(np.diff(g[:, 0]) > 0)
    c = g[:, 2:].copy().view(np.float32).astype(np.float64)
    y1, y2 = g[:, 1] & 0xFFFF, (g[:, 1] >> 16) & 0xFFFF
    A = np.zeros((y.shape[0], a_floats))
    A[:, g[:, 0]] = c[:, 0] * y[:, y1] + c[:, 1] * y[:, y2]
    return A


def _blocks(plan):
    nb, off_b, off_k = plan[1], plan[10], plan[11]
    blocks = plan[off_b:off_b + 4 * nb].reshape(nb, 4)
    klist = plan[off_k:off_k + plan[6]]
    base, out = 0, []
    for oo, rows, kb, K in blocks:
        out.append((oo, rows, klist[kb:kb + K], base))
        base += rows * K
    return out


def run_gemm(plan, y, xin, w, dout):
    """out[o] += A w[P] xin[xi] per block (kinds forward and dx)."""
    A = _A(plan, y)
    out = np.zeros((xin.shape[0], dout, xin.shape[2]))
    for oo, rows, kl, base in _blocks(plan):
        assert 1 <= rows <= 16  # the matrix cores' 16 rows (degree 8 split as 16 + 1)
        for k, ent in enumerate(kl):
            if ent < 0:
                continue
            P, xi = ent >> 16, ent & 0xFFFF
            a = A[:, base + k * rows: base + (k + 1) * rows]          # [B][rows]
            out[:, oo:oo + rows] += a[:, :, None] * (w[:, P] * xin[:, xi])[:, None, :]
    return out


def run_dw(plan, y, x, dz):
    """dw[P] = sum over the rows (P, M) of dz[o] (A x)[row]: tiles of four
    quads of rows stacked per x irrep (A stored with a row stride of 16),
    each quad one path's (16 t + rel) and each row naming its dz row."""
    A = _A(plan, y)
    nb, P, off_b, off_k, off_rt = plan[1], plan[5], plan[10], plan[11], plan[8]
    blocks = plan[off_b:off_b + 4 * nb].reshape(nb, 4)
    rowtab = plan[off_rt:off_rt + 16 * nb].reshape(nb, 16)
    dw = np.zeros((x.shape[0], P, x.shape[2]))
    base = 0
    for b, (t, rows, kb, K) in enumerate(blocks):
        assert 4 <= rows <= 16 and rows % 4 == 0 and K % 4 == 0 and K <= 16
        z = np.zeros((x.shape[0], 16, x.shape[2]))
        for k in range(K):
            ent = plan[off_k + kb + k]
            if ent >= 0:
                z += A[:, base + 16 * k: base + 16 * (k + 1), None] * x[:, ent][:, None, :]
        for r in range(16):
            e = rowtab[b, r]
            rel, o = e & 1023, e >> 10
            assert rel == rowtab[b, r - r % 4] & 1023  # one path per quad
            if r >= rows:
                assert e == 16
            if o == 0:  # a padding row: A stays zero there
                assert not A[:, base + r: base + 16 * K: 16].any()
                continue
            assert rel < 16
            dw[:, 16 * t + rel] += dz[:, o - 1] * z[:, r]
        base += 16 * K
    assert base == plan[9]
    return dw


def run_dy(plan, x, w, dz, dy_dim):
    """G[row][col] = sum_q w[P] own[q] col[q] over the slab rows [x; w; dz],
    then dy[yi] = sum of c G over yi's entries."""
    nb, off_b, off_r, off_yp, off_ye = plan[1], plan[10], plan[11], plan[12], plan[14]
    blocks = plan[off_b:off_b + 4 * nb].reshape(nb, 4)
    rows = plan[off_r:off_r + plan[6]]
    slab = np.concatenate([x, w, dz], axis=1)
    G = np.zeros((x.shape[0], rows.shape[0], 16))
    for co, ncol, r0, nr in blocks:
        assert 1 <= ncol <= 16 and nr % 16 == 0
        for r in range(r0, r0 + nr):
            if rows[r] < 0:
                continue
            P, own = rows[r] & 0xFFFF, rows[r] >> 16
            G[:, r, :ncol] = np.einsum("bq,bcq->bc", w[:, P] * slab[:, own], slab[:, co:co + ncol])
    yptr = plan[off_yp:off_yp + dy_dim + 1]
    ye = plan[off_ye:off_ye + 2 * yptr[-1]].reshape(-1, 2)
    cf = ye[:, 1].copy().view(np.float32).astype(np.float64)
    Gf = G.reshape(x.shape[0], -1)
    return np.stack([(Gf[:, ye[yptr[k]:yptr[k + 1], 0]] * cf[yptr[k]:yptr[k + 1]]).sum(axis=1)
                     for k in range(dy_dim)], axis=1)


def _case(L, skew=False, per_path=False, out=None, C=4, B=5, seed=0):
    xi = S.degree_irreps(L, skew)
    oi = out if out is not None else xi
    yi = S.sh_irreps(L)
    d = api.Desc(xi, yi, oi, C, api.E3_OUT_PER_PATH if per_path else 0)
    od = O.Desc(xi, yi, oi, C, per_path=per_path)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, d.dx, C))
    y = O.sh(L, rng.standard_normal((B, 3)))
    w = rng.standard_normal((B, api.num_paths(d), C))
    dz = rng.standard_normal((B, d.dout, C))
    return d, od, x, y, w, dz


CASES = [(1, False, False), (2, False, False), (3, True, False), (4, False, False),
         (5, False, True), (6, False, False), (6, True, False), (7, False, False),
         (7, True, False), (8, False, False), (8, True, False)]


@pytest.mark.parametrize("L,skew,pp", CASES)
def test_dense_plans_against_oracle(L, skew, pp):
    d, od, x, y, w, dz = _case(L, skew, pp, seed=L)
    z = run_gemm(_plan(d, api.E3_GEN_GEMM), y, x, w, d.dout)
    np.testing.assert_allclose(z, O.tp_forward(od, x, y, w), atol=1e-5, rtol=1e-5)
    rdx, rdw, rdy = O.tp_backward(od, x, y, w, dz)
    dx = run_gemm(_plan(d, api.E3_GEN_GEMM_DX), y, dz, w, d.dx)
    np.testing.assert_allclose(dx, rdx, atol=1e-5, rtol=1e-5)
    dw = run_dw(_plan(d, api.E3_GEN_GEMM_DW), y, x, dz)
    np.testing.assert_allclose(dw, rdw, atol=1e-5, rtol=1e-5)
    dy = run_dy(_plan(d, api.E3_GEN_GEMM_DY), x, w, dz, d.dy)
    np.testing.assert_allclose(dy, rdy, atol=1e-4, rtol=1e-5)


def test_dense_plans_pathless_output_block():
    d, od, x, y, w, dz = _case(1, out=[(0, 1), (1, -1), (0, -1)], seed=9)
    z = run_gemm(_plan(d, api.E3_GEN_GEMM), y, x, w, d.dout)
    np.testing.assert_allclose(z, O.tp_forward(od, x, y, w), atol=1e-6)
    rdx, rdw, rdy = O.tp_backward(od, x, y, w, dz)
    np.testing.assert_allclose(run_gemm(_plan(d, api.E3_GEN_GEMM_DX), y, dz, w, d.dx), rdx, atol=1e-6)
    np.testing.assert_allclose(run_dw(_plan(d, api.E3_GEN_GEMM_DW), y, x, dz), rdw, atol=1e-6)
    np.testing.assert_allclose(run_dy(_plan(d, api.E3_GEN_GEMM_DY), x, w, dz, d.dy), rdy, atol=1e-5)
