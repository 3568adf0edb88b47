"""Python front of the fp64 CPU oracle (oracle/e3_oracle.c), via ctypes.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  It shares
no code with the HIP library (``clebsch_gordan_tensor_amd``): irreps are
passed here as plain lists of ``(l, parity)`` and every array is float64.

What each function computes, and the passage it follows, is stated in the C
file next to the function it wraps.  Where a result has a plain definition
(the convolution and tensor product of the e3j paper, E.1 Eq.10-13 and
Eq.16), the oracle is that definition written out as loops.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libe3oracle.so")
_MAX_IRREPS = 16

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from oracle.build import build_oracle  # builds only when nothing is built
        build_oracle()
    lib = C.CDLL(_LIB_PATH)
    dp = C.POINTER(C.c_double)
    ip = C.POINTER(C.c_int)
    lp = C.POINTER(C.c_int64)
    lib.oracle_cg_complex.restype = C.c_double
    lib.oracle_cg_complex.argtypes = [C.c_int] * 6
    lib.oracle_cg_real.restype = C.c_int
    lib.oracle_cg_real.argtypes = [C.c_int, C.c_int, C.c_int, dp]
    lib.oracle_umat.restype = None
    lib.oracle_umat.argtypes = [C.c_int, dp, dp]
    lib.oracle_sh_batch.restype = C.c_int
    lib.oracle_sh_batch.argtypes = [C.c_int, C.c_int64, dp, dp]
    lib.oracle_sh_general.argtypes = [C.c_int, dp, dp]
    lib.oracle_num_threads.restype = C.c_int
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [C.c_int]
    lib.oracle_num_paths.restype = C.c_int
    lib.oracle_num_paths.argtypes = [C.c_void_p]
    lib.oracle_path_info.restype = C.c_int
    lib.oracle_path_info.argtypes = [C.c_void_p, C.c_int, ip, ip, ip]
    lib.oracle_conv_forward.restype = C.c_int
    lib.oracle_conv_forward.argtypes = [C.c_void_p, C.c_int, C.c_int64, ip, ip, dp, dp, dp, dp,
                                        C.c_int, ip, dp]
    lib.oracle_tp_forward.restype = C.c_int
    lib.oracle_tp_forward.argtypes = [C.c_void_p, C.c_int64, dp, dp, dp, C.c_int, lp, dp]
    lib.oracle_conv_backward_dx.restype = C.c_int
    lib.oracle_conv_backward_dx.argtypes = [C.c_void_p, C.c_int, C.c_int64, ip, ip, dp, dp, dp,
                                            dp, C.c_int, ip, dp]
    lib.oracle_conv_backward_edge.restype = C.c_int
    lib.oracle_conv_backward_edge.argtypes = [C.c_void_p, C.c_int, C.c_int64, ip, ip, dp, dp,
                                              dp, dp, dp, C.c_int, lp, dp, dp]
    lib.oracle_tp_backward.restype = C.c_int
    lib.oracle_tp_backward.argtypes = [C.c_void_p, C.c_int64, dp, dp, dp, dp, C.c_int, lp, dp,
                                       dp, dp]
    lib.oracle_sh_grad_batch.restype = C.c_int
    lib.oracle_sh_grad_batch.argtypes = [C.c_int, C.c_int64, dp, dp, dp]
    lib.oracle_edge_grad_to_nodes.restype = C.c_int
    lib.oracle_edge_grad_to_nodes.argtypes = [C.c_int, C.c_int64, ip, ip, dp, dp]
    lib.oracle_linear.restype = C.c_int
    lib.oracle_linear.argtypes = [C.c_int, ip, ip, C.c_int, C.c_int, ip, ip, C.c_int, C.c_int64,
                                  dp, dp, dp]
    lib.oracle_linear_backward.restype = C.c_int
    lib.oracle_linear_backward.argtypes = [C.c_int, ip, ip, C.c_int, C.c_int, ip, ip, C.c_int,
                                           C.c_int64, dp, dp, dp, dp, dp]
    _lib = lib
    return lib


class _CDesc(C.Structure):
    _fields_ = [("nx", C.c_int), ("ny", C.c_int), ("no", C.c_int),
                ("xl", C.c_int * _MAX_IRREPS), ("xp", C.c_int * _MAX_IRREPS),
                ("yl", C.c_int * _MAX_IRREPS), ("yp", C.c_int * _MAX_IRREPS),
                ("ol", C.c_int * _MAX_IRREPS), ("op", C.c_int * _MAX_IRREPS),
                ("C", C.c_int), ("per_path", C.c_int)]


def parse_irreps(s: str):
    """'128x0e+128x1o' -> (mul, [(0, 1), (1, -1)]); every mul must agree."""
    out, muls = [], set()
    for term in s.replace(" ", "").split("+"):
        if "x" in term:
            mul, ir = term.split("x")
            muls.add(int(mul))
        else:
            ir = term
            muls.add(1)
        l, p = int(ir[:-1]), {"e": 1, "o": -1}[ir[-1]]
        out.append((l, p))
    if len(muls) != 1:
        raise ValueError("channel-wise irreps need one multiplicity: " + s)
    return muls.pop(), out


class Desc:
    """Irreps of x, y and the output, as lists of (l, parity), and C channels;
    per_path: one output block per path (path order) instead of one per
    output irrep."""

    def __init__(self, x, y, out, channels, per_path=False):
        self.x, self.y, self.out, self.C = list(x), list(y), list(out), int(channels)
        self.per_path = bool(per_path)
        c = _CDesc()
        c.nx, c.ny, c.no, c.C = len(self.x), len(self.y), len(self.out), self.C
        c.per_path = int(self.per_path)
        for arr_l, arr_p, ir in ((c.xl, c.xp, self.x), (c.yl, c.yp, self.y),
                                 (c.ol, c.op, self.out)):
            if len(ir) > _MAX_IRREPS:
                raise ValueError("too many irreps")
            for i, (l, p) in enumerate(ir):
                arr_l[i], arr_p[i] = l, p
        self._c = c

    @property
    def dx(self):
        return sum(2 * l + 1 for l, _ in self.x)

    @property
    def dy(self):
        return sum(2 * l + 1 for l, _ in self.y)

    @property
    def dout(self):
        if self.per_path:
            return sum(2 * self.out[o][0] + 1 for _, _, o in paths(self))
        return sum(2 * l + 1 for l, _ in self.out)

    def ptr(self):
        return C.byref(self._c)


def _dp(a):
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _ip(a):
    return a.ctypes.data_as(C.POINTER(C.c_int))


def _lp(a):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (results do not
    depend on it)."""
    _load().oracle_set_num_threads(int(n))


def num_threads() -> int:
    return _load().oracle_num_threads()


def cg_complex(l1, m1, l2, m2, L, M) -> float:
    return _load().oracle_cg_complex(l1, m1, l2, m2, L, M)


def cg_real(l1, l2, L) -> np.ndarray:
    out = np.zeros((2 * L + 1) * (2 * l1 + 1) * (2 * l2 + 1))
    if _load().oracle_cg_real(l1, l2, L, _dp(out)) != 0:
        raise ValueError("uncoupled triple")
    return out.reshape(2 * L + 1, 2 * l1 + 1, 2 * l2 + 1)


def umat(l) -> np.ndarray:
    n = 2 * l + 1
    re, im = np.zeros(n * n), np.zeros(n * n)
    _load().oracle_umat(l, _dp(re), _dp(im))
    return (re + 1j * im).reshape(n, n)


def sh(lmax: int, vecs) -> np.ndarray:
    v = _f64(vecs).reshape(-1, 3)
    out = np.zeros((v.shape[0], (lmax + 1) ** 2))
    if _load().oracle_sh_batch(lmax, v.shape[0], _dp(v), _dp(out)) != 0:
        raise ValueError("lmax out of range")
    return out


def num_paths(d: Desc) -> int:
    return _load().oracle_num_paths(d.ptr())


def paths(d: Desc):
    lib = _load()
    res = []
    for i in range(num_paths(d)):
        a, b, c = C.c_int(), C.c_int(), C.c_int()
        lib.oracle_path_info(d.ptr(), i, C.byref(a), C.byref(b), C.byref(c))
        res.append((a.value, b.value, c.value))
    return res


def _y_args(evec, Y):
    if (evec is None) == (Y is None):
        raise ValueError("give exactly one of evec, Y")
    ev = _f64(evec) if evec is not None else None
    yy = _f64(Y) if Y is not None else None
    return ev, yy


def conv_forward(d: Desc, rowptr, sender, x, w, evec=None, Y=None, rows=None):
    """m[rows] (all receivers by default), shape [len(rows)][dout][C]."""
    rowptr, sender = _i32(rowptr), _i32(sender)
    n_nodes = rowptr.shape[0] - 1
    rows = np.arange(n_nodes, dtype=np.int32) if rows is None else _i32(rows)
    ev, yy = _y_args(evec, Y)
    x, w = _f64(x), _f64(w)
    m = np.zeros((rows.shape[0], d.dout, d.C))
    r = _load().oracle_conv_forward(d.ptr(), n_nodes, sender.shape[0], _ip(rowptr), _ip(sender),
                                    _dp(ev) if ev is not None else None,
                                    _dp(yy) if yy is not None else None, _dp(x), _dp(w),
                                    rows.shape[0], _ip(rows), _dp(m))
    if r != 0:
        raise ValueError("oracle_conv_forward rejected its arguments")
    return m


def tp_forward(d: Desc, x, y, w, rows=None):
    """z[rows] (all rows by default), shape [len(rows)][dout][C]."""
    x, y, w = _f64(x), _f64(y), _f64(w)
    n = x.shape[0]
    rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    z = np.zeros((rows.shape[0], d.dout, d.C))
    r = _load().oracle_tp_forward(d.ptr(), n, _dp(x), _dp(y), _dp(w), rows.shape[0], _lp(rows),
                                  _dp(z))
    if r != 0:
        raise ValueError("oracle_tp_forward rejected its arguments")
    return z


def conv_backward_dx(d: Desc, rowptr, sender, w, dm, evec=None, Y=None, rows=None):
    """dx[rows] (all senders by default), shape [len(rows)][dx][C]."""
    rowptr, sender = _i32(rowptr), _i32(sender)
    n_nodes = rowptr.shape[0] - 1
    rows = np.arange(n_nodes, dtype=np.int32) if rows is None else _i32(rows)
    ev, yy = _y_args(evec, Y)
    w, dm = _f64(w), _f64(dm)
    dx = np.zeros((rows.shape[0], d.dx, d.C))
    r = _load().oracle_conv_backward_dx(d.ptr(), n_nodes, sender.shape[0], _ip(rowptr),
                                        _ip(sender), _dp(ev) if ev is not None else None,
                                        _dp(yy) if yy is not None else None, _dp(w), _dp(dm),
                                        rows.shape[0], _ip(rows), _dp(dx))
    if r != 0:
        raise ValueError("oracle_conv_backward_dx rejected its arguments")
    return dx


def conv_backward_edge(d: Desc, rowptr, sender, x, w, dm, evec=None, Y=None, edges=None):
    """(dw[edges] [len][P][C], dY[edges] [len][dy]); all edges by default."""
    rowptr, sender = _i32(rowptr), _i32(sender)
    n_nodes = rowptr.shape[0] - 1
    n_edges = sender.shape[0]
    edges = (np.arange(n_edges, dtype=np.int64) if edges is None
             else np.ascontiguousarray(edges, np.int64))
    ev, yy = _y_args(evec, Y)
    x, w, dm = _f64(x), _f64(w), _f64(dm)
    P = num_paths(d)
    dw = np.zeros((edges.shape[0], P, d.C))
    dY = np.zeros((edges.shape[0], d.dy))
    r = _load().oracle_conv_backward_edge(d.ptr(), n_nodes, n_edges, _ip(rowptr), _ip(sender),
                                          _dp(ev) if ev is not None else None,
                                          _dp(yy) if yy is not None else None, _dp(x), _dp(w),
                                          _dp(dm), edges.shape[0], _lp(edges), _dp(dw), _dp(dY))
    if r != 0:
        raise ValueError("oracle_conv_backward_edge rejected its arguments")
    return dw, dY


def tp_backward(d: Desc, x, y, w, dz, rows=None):
    """(dx, dw, dy) of the batched TP for the cotangent dz, at rows (all by
    default): shapes [len][dx][C], [len][P][C], [len][dy]."""
    x, y, w, dz = _f64(x), _f64(y), _f64(w), _f64(dz)
    n = x.shape[0]
    rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    P = num_paths(d)
    dx = np.zeros((rows.shape[0], d.dx, d.C))
    dw = np.zeros((rows.shape[0], P, d.C))
    dy = np.zeros((rows.shape[0], d.dy))
    r = _load().oracle_tp_backward(d.ptr(), n, _dp(x), _dp(y), _dp(w), _dp(dz), rows.shape[0],
                                   _lp(rows), _dp(dx), _dp(dw), _dp(dy))
    if r != 0:
        raise ValueError("oracle_tp_backward rejected its arguments")
    return dx, dw, dy


def sh_general(l: int, vecs) -> np.ndarray:
    """Degree-l harmonics by the oracle's general (Legendre) construction,
    [n][2l+1]; sh() uses it for l >= 4 and closed-form polynomials below."""
    v = _f64(vecs).reshape(-1, 3)
    out = np.zeros((v.shape[0], 2 * l + 1))
    for i in range(v.shape[0]):
        if _load().oracle_sh_general(l, _dp(v[i]), _dp(out[i])) != 0:
            raise ValueError("degree out of range")
    return out


def sh_grad(lmax: int, vecs, dY) -> np.ndarray:
    """Vector gradient J^T dY of the harmonics of vecs [n][3], dY [n][(lmax+1)^2]."""
    v = _f64(vecs).reshape(-1, 3)
    g = _f64(dY).reshape(v.shape[0], (lmax + 1) ** 2)
    out = np.zeros((v.shape[0], 3))
    if _load().oracle_sh_grad_batch(lmax, v.shape[0], _dp(v), _dp(g), _dp(out)) != 0:
        raise ValueError("lmax out of range")
    return out


def sh_grad_fd(lmax: int, vecs, dY) -> np.ndarray:
    """J^T dY of the harmonics of vecs [n][3] by fourth-order central
    differences of sh() (fp64), for the degrees (4..8) that the closed-form
    partials of sh_grad do not cover.  Step h = 1e-3 |r| per axis: the
    truncation error is O(h^4 |d^5 Y|), about 1e-9 of the value at l = 6
    and 3e-8 at l = 8, and the rounding error about 1e-13 |Y| / h.  A zero
    vector gets 0."""
    v = _f64(vecs).reshape(-1, 3)
    g = _f64(dY).reshape(v.shape[0], (lmax + 1) ** 2)
    r = np.linalg.norm(v, axis=1)
    h = 1e-3 * np.where(r > 0, r, 1.0)
    out = np.zeros((v.shape[0], 3))
    for k in range(3):
        e = np.zeros_like(v)
        e[:, k] = h

        def f(s):
            return (sh(lmax, v + s * e) * g).sum(axis=1)

        out[:, k] = (-f(2) + 8 * f(1) - 8 * f(-1) + f(-2)) / (12 * h)
    out[r == 0] = 0.0
    return out


def edge_grad_to_nodes(rowptr, sender, g) -> np.ndarray:
    """dpos [N][3] from edge-vector gradients g [E][3] (r_e = pos[recv] - pos[sender])."""
    rowptr, sender = _i32(rowptr), _i32(sender)
    g = _f64(g).reshape(sender.shape[0], 3)
    n = rowptr.shape[0] - 1
    out = np.zeros((n, 3))
    if _load().oracle_edge_grad_to_nodes(n, sender.shape[0], _ip(rowptr), _ip(sender), _dp(g),
                                         _dp(out)) != 0:
        raise ValueError("oracle_edge_grad_to_nodes rejected its arguments")
    return out


def _lp_arrays(irreps):
    ls = np.ascontiguousarray([l for l, _ in irreps], dtype=np.int32)
    ps = np.ascontiguousarray([p for _, p in irreps], dtype=np.int32)
    return ls, ps


def linear_num_weights(in_irreps, out_irreps) -> int:
    """Number of Cin x Cout weight matrices of the channel mixing."""
    il, ip_ = _lp_arrays(in_irreps)
    ol, op_ = _lp_arrays(out_irreps)
    n = _load().oracle_linear(len(il), _ip(il), _ip(ip_), 1, len(ol), _ip(ol), _ip(op_), 1, 0,
                              None, None, None)
    if n < 0:
        raise ValueError("oracle_linear rejected the irreps")
    return n


def linear(in_irreps, out_irreps, x, W):
    """y [rows][dout][Cout] of the per-irrep channel mixing; x [rows][din][Cin],
    W [n_pairs][Cin][Cout]."""
    x, W = _f64(x), _f64(W)
    il, ip_ = _lp_arrays(in_irreps)
    ol, op_ = _lp_arrays(out_irreps)
    rows, din, cin = x.shape
    cout = W.shape[-1]
    dout = sum(2 * l + 1 for l, _ in out_irreps)
    y = np.zeros((rows, dout, cout))
    n = _load().oracle_linear(len(il), _ip(il), _ip(ip_), cin, len(ol), _ip(ol), _ip(op_), cout,
                              rows, _dp(x), _dp(W), _dp(y))
    if n < 0:
        raise ValueError("oracle_linear rejected its arguments")
    return y


def linear_backward(in_irreps, out_irreps, x, W, dy):
    """(dx [rows][din][Cin], dW [n_pairs][Cin][Cout]) of the channel mixing."""
    x, W, dy = _f64(x), _f64(W), _f64(dy)
    il, ip_ = _lp_arrays(in_irreps)
    ol, op_ = _lp_arrays(out_irreps)
    rows, din, cin = x.shape
    cout = W.shape[-1]
    dx = np.zeros_like(x)
    dW = np.zeros_like(W)
    n = _load().oracle_linear_backward(len(il), _ip(il), _ip(ip_), cin, len(ol), _ip(ol),
                                       _ip(op_), cout, rows, _dp(x), _dp(W), _dp(dy), _dp(dx),
                                       _dp(dW))
    if n < 0:
        raise ValueError("oracle_linear_backward rejected its arguments")
    return dx, dW


def conv_double_backward(d: Desc, rowptr, sender, Y, x, w, dm, ddx, ddY, ddw):
    """Double backward of the convolution in the given-harmonics form (e3j
    E.1 Eq.17-18): for variations (ddx, ddY, ddw) of the backward's outputs
    (dx, dY, dw), the variations of its inputs

      ddm = conv(ddx, Y, w) + conv(x, ddY, w) + conv(x, Y, ddw)
      dx2 = [dx of conv_bwd(x, ddY, w, dm)] + [dx of conv_bwd(x, Y, ddw, dm)]
      dY2 = [dY of conv_bwd(ddx, Y, w, dm)] + [dY of conv_bwd(x, Y, ddw, dm)]
      dw2 = [dw of conv_bwd(ddx, Y, w, dm)] + [dw of conv_bwd(x, ddY, w, dm)]

    composed from this module's convolution and its backward, in the pages'
    order.  Returns (dx2, dY2, dw2, ddm)."""
    fwd = lambda x_, Y_, w_: conv_forward(d, rowptr, sender, x_, w_, Y=Y_)
    bdx = lambda Y_, w_: conv_backward_dx(d, rowptr, sender, w_, dm, Y=Y_)
    bed = lambda x_, Y_, w_: conv_backward_edge(d, rowptr, sender, x_, w_, dm, Y=Y_)
    ddm = fwd(ddx, Y, w) + fwd(x, ddY, w) + fwd(x, Y, ddw)
    dx2 = bdx(ddY, w) + bdx(Y, ddw)
    dwa, dYa = bed(ddx, Y, w)
    dwb, _ = bed(x, ddY, w)
    _, dYc = bed(x, Y, ddw)
    return dx2, dYa + dYc, dwa + dwb, ddm
