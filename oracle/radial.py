"""fp64 CPU oracle of the radial edge weights and of the convolution that
computes them on the fly.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this module.  It shares
no code with the HIP library.

The e3j paper (A.3, the edge scalars s_ab of Eq.7; E.1, "Message weighting
with edge scalars") takes the per-edge, per-path, per-channel weights from
an MLP applied to a radial basis embedding of the distance |r_ab|; its model
table (Table 3) uses 8 radial basis functions.  The pages fix nothing else,
so the plainest reading is taken and written out here:

    B_n(d) = sqrt(2 / r_c) sin(n pi d / r_c) / d,           n = 1 .. n_basis
    h_k    = silu(sum_n B_n(d) W1[n][k]),  silu(t) = t / (1 + exp(-t))
    w[j]   = sum_k h_k W2[k][j],                            j < P * C

(no envelope, no biases; at d = 0 the basis takes its limit n pi / r_c *
sqrt(2 / r_c)).  The weights feed the convolution of e3j A.3 Eq.7 / E.1
Eq.12-13 exactly as a given w[E][P][C] does.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O


def bessel_basis(d, cutoff: float, n_basis: int) -> np.ndarray:
    """[E][n_basis] radial basis of the distances d (fp64)."""
    d = np.asarray(d, dtype=np.float64)
    n = np.arange(1, n_basis + 1, dtype=np.float64)
    pref = np.sqrt(2.0 / cutoff)
    arg = np.pi * np.outer(d, n) / cutoff
    out = np.empty_like(arg)
    nz = d != 0.0
    out[nz] = pref * np.sin(arg[nz]) / d[nz, None]
    out[~nz] = pref * np.pi * n / cutoff
    return out


def bessel_basis_deriv(d, cutoff: float, n_basis: int) -> np.ndarray:
    """dB_n/dd, [E][n_basis] (the derivative of the quotient written out)."""
    d = np.asarray(d, dtype=np.float64)
    n = np.arange(1, n_basis + 1, dtype=np.float64)
    pref = np.sqrt(2.0 / cutoff)
    k = np.pi * n / cutoff
    arg = np.outer(d, k)
    out = np.zeros_like(arg)
    nz = d != 0.0
    dd = d[nz, None]
    out[nz] = pref * (k * np.cos(arg[nz]) / dd - np.sin(arg[nz]) / dd ** 2)
    return out  # the limit at d = 0 is 0 (the basis is even in d)


def silu(t):
    return t / (1.0 + np.exp(-t))


def silu_deriv(t):
    s = 1.0 / (1.0 + np.exp(-t))
    return s * (1.0 + t * (1.0 - s))


def _distances(evec):
    return np.linalg.norm(np.asarray(evec, dtype=np.float64), axis=1)


def radial_mlp(evec, cutoff: float, W1, W2) -> np.ndarray:
    """w[E][ncols] = silu(B(|r|) W1) W2, in fp64."""
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    B = bessel_basis(_distances(evec), cutoff, W1.shape[0])
    return silu(B @ W1) @ W2


def radial_mlp_backward(evec, cutoff: float, W1, W2, dw):
    """Cotangents of radial_mlp: (dW1, dW2, dvec) for the output cotangent dw
    [E][ncols]; dvec[e] = (dL/dd_e) r_e / |r_e| (the weights depend on the
    edge vector through its length only)."""
    evec = np.asarray(evec, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    d = _distances(evec)
    B = bessel_basis(d, cutoff, W1.shape[0])
    pre = B @ W1
    h = silu(pre)
    dW2 = h.T @ dw
    dh = dw @ W2.T
    dpre = dh * silu_deriv(pre)
    dW1 = B.T @ dpre
    dB = dpre @ W1.T
    dd = np.sum(dB * bessel_basis_deriv(d, cutoff, W1.shape[0]), axis=1)
    unit = np.zeros_like(evec)
    nz = d > 0
    unit[nz] = evec[nz] / d[nz, None]
    return dW1, dW2, dd[:, None] * unit


def conv_forward_radial(desc, rowptr, sender, evec, x, cutoff: float, W1, W2, rows=None):
    """The convolution of e3j A.3 Eq.7 with w = radial_mlp(evec): m[rows]
    (all receivers by default), [len(rows)][dout][C].  With a row sample only
    the edges of the sampled receivers are weighted (the others get empty
    segments), so full-size graphs stay cheap."""
    rowptr = np.asarray(rowptr, dtype=np.int64)
    sender = np.asarray(sender)
    evec = np.asarray(evec)
    P = O.num_paths(desc)
    n = rowptr.shape[0] - 1
    if rows is None:
        E = sender.shape[0]
        w = radial_mlp(evec, cutoff, W1, W2).reshape(E, P, desc.C)
        return O.conv_forward(desc, rowptr, sender, x, w, evec=evec)
    rows = np.asarray(rows, dtype=np.int64)
    keep = np.unique(rows)
    counts = np.zeros(n, dtype=np.int64)
    counts[keep] = rowptr[keep + 1] - rowptr[keep]
    sub_ptr = np.concatenate([[0], np.cumsum(counts)])
    idx = np.concatenate([np.arange(rowptr[b], rowptr[b + 1]) for b in keep]).astype(np.int64)
    w = radial_mlp(evec[idx], cutoff, W1, W2).reshape(idx.shape[0], P, desc.C)
    return O.conv_forward(desc, sub_ptr, sender[idx], x, w, evec=evec[idx], rows=rows)
