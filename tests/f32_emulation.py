"""Float32 emulation of the specialised forward convolution kernel's
arithmetic, in its order, on the CPU (test infrastructure: it explains and
pins the float32 rounding floor of a workload, it is not the oracle).

What it reproduces, per receiver:
  - the harmonics of each edge vector are the float32 values nearest to the
    exact ones (the kernel evaluates them in fp64 and rounds once; here the
    oracle's fp64 harmonics are rounded);
  - per path, the CG sum over m2 for each (M, m1) pair, A = c Y (fma for
    further records), with c the float32-rounded coefficient;
  - contract-then-weight when 2l1+1 < 2L+1 (u = w x, then acc += A u by
    fma), else weight-then-contract (z = sum A x by fma, then acc += w z);
  - the edges of a receiver split over `groups` edge groups (edge k to group
    k mod groups), each with its own accumulator, the groups added at the
    end (64 / G groups per wavefront, G = C / channels-per-lane lanes).
Fused multiply-adds are emulated as an fp64 product-sum rounded once to
float32 (exact but for double rounding in rare ties).

The coefficients are the library's own real CG blocks (e3_cg_block): the
emulation stands for the kernel, so it uses the kernel's table.
"""
from __future__ import annotations

import numpy as np

from clebsch_gordan_tensor_amd import api
from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O

f32 = np.float32


def _fma(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(f32)


def _blocks(p, per_path):
    xo = np.cumsum([0] + [2 * l + 1 for l, _ in p.x_irreps])
    yo = np.cumsum([0] + [2 * l + 1 for l, _ in p.y_irreps])
    ooff = np.cumsum([0] + [2 * l + 1 for l, _ in p.out_irreps])
    out, opp = [], 0
    for (i, j, k) in S.path_list(p.x_irreps, p.y_irreps, p.out_irreps):
        l1, l2, L = p.x_irreps[i][0], p.y_irreps[j][0], p.out_irreps[k][0]
        cb = api.cg_block(l1, l2, L)
        recs = [(M, m1, m2, f32(cb[M, m1, m2])) for M in range(2 * L + 1)
                for m1 in range(2 * l1 + 1) for m2 in range(2 * l2 + 1)
                if abs(cb[M, m1, m2]) > 1e-12]
        out.append((l1, L, int(xo[i]), int(yo[j]), recs, opp if per_path else int(ooff[k])))
        opp += 2 * L + 1
    return out


def conv_forward_f32(p, per_path: bool, groups: int, lmax_y: int = 3) -> np.ndarray:
    """m [N][dout][C] as the kernel computes it in float32."""
    g = p.graph
    Y = O.sh(lmax_y, g.evec.astype(np.float64)).astype(f32)
    blocks = _blocks(p, per_path)
    dout = blocks[-1][5] + 2 * blocks[-1][1] + 1 if per_path else S.dim(p.out_irreps)
    N, C = g.n_nodes, p.channels
    deg = np.diff(g.rowptr)
    accs = np.zeros((groups, N, dout, C), f32)
    for k in range(int(deg.max()) if N else 0):
        bs = np.flatnonzero(deg > k)
        e = g.rowptr[bs] + k
        acc = accs[k % groups][bs]
        xs, ws = p.x[g.sender[e]], p.w[e]
        for pi, (l1, L, xo, yo, recs, oo) in enumerate(blocks):
            n1, nL = 2 * l1 + 1, 2 * L + 1

            def pairs():
                prev = None
                for r, (M, m1, m2, c) in enumerate(recs):
                    yv = Y[e, yo + m2]
                    A = (c * yv).astype(f32) if prev != (M, m1) else _fma(c, yv, A)
                    prev = (M, m1)
                    if r == len(recs) - 1 or recs[r + 1][:2] != (M, m1):
                        yield M, m1, A

            if n1 < nL:
                u = (ws[:, pi, None, :] * xs[:, xo:xo + n1, :]).astype(f32)
                for M, m1, A in pairs():
                    acc[:, oo + M] = _fma(A[:, None], u[:, m1], acc[:, oo + M])
            else:
                z = np.zeros((len(bs), nL, C), f32)
                for M, m1, A in pairs():
                    z[:, M] = _fma(A[:, None], xs[:, xo + m1], z[:, M])
                for M in range(nL):
                    acc[:, oo + M] = _fma(ws[:, pi], z[:, M], acc[:, oo + M])
        accs[k % groups][bs] = acc
    m = accs[0]
    for gi in range(1, groups):
        m = (m + accs[gi]).astype(f32)
    return m
