"""Seeded synthetic inputs for the equivariant convolution and tensor product.

This module is the only code that both the HIP path and the CPU oracle take
inputs from.  It holds no harmonics, no Clebsch-Gordan coefficients and no
contraction: only positions, neighbour lists, CSR sorting and random draws
(plus, for the water box, the random radial MLP that stands in for trained
edge weights).

The workloads follow the MLIP setting of the e3j paper (section 3.1.2 and
Table 3: 128 channels, l_max 3, 5 A cutoff, radial basis of 8 functions) and
of its Table 1 (about 45 neighbours per node):

  tiny      64 nodes, 6 A cube, cutoff 3 A, 8x(0e+1o) -> 8x(0e+1o), SH l <= 1
  tp        200,000 independent rows, 128x(0e+1o+2e) (x) SH l <= 3 -> 128x(0e+1o+2e+3o)
  water3k   3,000 atoms at 0.1 atoms/A^3, cutoff 5 A, 128x(0e+1o) -> 128x(0e+1o+2e+3o),
            weights from a random 2-layer radial MLP on 8 Bessel functions
  mace64k   64,000 atoms at 0.1 atoms/A^3, cutoff 5 A, same irreps, N(0,1) weights
  ho20k     20,000 atoms, node labels randomly permuted, 64x(0e+1o+2e+3o) both
            sides, bf16 storage
  deg<L>    (make_conv_degree) the higher-degree convolution of e3j B.1 Fig 7:
            2,048 nodes, about 45 neighbours (26.75 A cube, cutoff 5 A),
            128 channels, every irrep 0..L once on x and out, SH l <= L

Graph rule: ordered pairs (a -> b), a != b, |pos_b - pos_a| <= cutoff, open
cube (no periodic images), edges sorted by (receiver, sender); the edge vector
is r = pos[receiver] - pos[sender].

Random draws: every array has its own PCG64 stream, derived from
SeedSequence((seed, tag)); large arrays are drawn in fixed chunks of rows,
chunk k from the k-th spawned child, so the values do not depend on thread
count.  bf16 storage rounds the fp32 draw to nearest-even.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------- irreps

_PARITY = {"e": 1, "o": -1}


def parse_irreps(s: str):
    """'128x0e+128x1o' -> (128, [(0, 1), (1, -1)]).  All multiplicities must
    agree (channel-wise product); a bare irrep has multiplicity 1."""
    out, muls = [], set()
    for term in s.replace(" ", "").split("+"):
        if "x" in term:
            mul, ir = term.split("x")
            muls.add(int(mul))
        else:
            ir = term
            muls.add(1)
        out.append((int(ir[:-1]), _PARITY[ir[-1]]))
    if len(muls) != 1:
        raise ValueError("channel-wise irreps need one multiplicity: " + s)
    return muls.pop(), out


def sh_irreps(lmax: int):
    """Irreps of the harmonic bank Y_0..Y_lmax: l with parity (-1)^l."""
    return [(l, 1 if l % 2 == 0 else -1) for l in range(lmax + 1)]


def dim(irreps):
    return sum(2 * l + 1 for l, _ in irreps)


def path_list(x, y, out):
    """Paths (ix, iy, io) in canonical order: x irrep, then y irrep, then
    output irrep; triangle rule and p_x p_y = p_out (parity rule of the e3j
    paper, B.1).  Used to shape inputs (w has one slot per path)."""
    res = []
    for i, (lx, px) in enumerate(x):
        for j, (ly, py) in enumerate(y):
            for k, (lo, po) in enumerate(out):
                if abs(lx - ly) <= lo <= lx + ly and px * py == po:
                    res.append((i, j, k))
    return res


def num_paths(x, y, out):
    return len(path_list(x, y, out))


# ---------------------------------------------------------------- draws

_CHUNK = 1 << 14


def _stream(seed: int, tag: int):
    return np.random.SeedSequence((int(seed), int(tag)))


def normal(shape, seed: int, tag: int, threads: int | None = None) -> np.ndarray:
    """N(0,1) float32 array; rows (first axis) drawn in chunks of 16384 rows,
    chunk k from child k of SeedSequence((seed, tag))."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    n = shape[0]
    if n == 0:
        return out
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = _stream(seed, tag).spawn(nch)

    def fill(k):
        lo, hi = k * _CHUNK, min(n, (k + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[k]))
        out[lo:hi] = g.standard_normal((hi - lo,) + shape[1:], dtype=np.float32)

    threads = threads or min(16, os.cpu_count() or 1)
    if nch == 1 or threads == 1:
        for k in range(nch):
            fill(k)
    else:
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nch)))
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 value (ties to even), returned as
    float32 holding exactly representable values (NaN is not expected)."""
    src = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    out = np.empty_like(src)
    ui, uo = src.view(np.uint32), out.view(np.uint32)
    step = 1 << 22

    def work(lo):
        u = ui[lo:lo + step]
        t = np.right_shift(u, np.uint32(16))
        np.bitwise_and(t, np.uint32(1), out=t)
        np.add(t, np.uint32(0x7FFF), out=t)
        np.add(t, u, out=t)
        np.bitwise_and(t, np.uint32(0xFFFF0000), out=uo[lo:lo + step])

    starts = range(0, src.shape[0], step)
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(work, starts))
    return out.reshape(np.shape(a))


# ---------------------------------------------------------------- graphs

@dataclass
class Graph:
    pos: np.ndarray      # [N, 3] float64
    rowptr: np.ndarray   # [N+1] int32, CSR by receiver
    sender: np.ndarray   # [E] int32
    receiver: np.ndarray  # [E] int32 (implied by rowptr; kept for convenience)
    evec: np.ndarray     # [E, 3] float32, pos[receiver] - pos[sender]

    @property
    def n_nodes(self):
        return int(self.rowptr.shape[0] - 1)

    @property
    def n_edges(self):
        return int(self.sender.shape[0])


def radius_graph(pos: np.ndarray, cutoff: float) -> Graph:
    from scipy.spatial import cKDTree

    n = pos.shape[0]
    pairs = cKDTree(pos).query_pairs(cutoff, output_type="ndarray")  # i < j, d <= cutoff
    if pairs.size == 0:
        pairs = np.zeros((0, 2), dtype=np.int64)
    snd = np.concatenate([pairs[:, 0], pairs[:, 1]]).astype(np.int64)
    rcv = np.concatenate([pairs[:, 1], pairs[:, 0]]).astype(np.int64)
    order = np.lexsort((snd, rcv))  # by receiver, then sender
    snd, rcv = snd[order], rcv[order]
    counts = np.bincount(rcv, minlength=n)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=rowptr[1:])
    if rowptr[-1] >= 2 ** 31:
        raise ValueError("edge count exceeds int32 indexing")
    evec = (pos[rcv] - pos[snd]).astype(np.float32)
    return Graph(pos=pos, rowptr=rowptr.astype(np.int32), sender=snd.astype(np.int32),
                 receiver=rcv.astype(np.int32), evec=evec)


def subgraph(g: Graph, ids):
    """Edges ids of g (kept in receiver order) as a CSR over all g's nodes:
    (rowptr, sender, evec, sorted ids).  Used to hand a sample of a large
    graph to a checker."""
    ids = np.sort(np.asarray(ids, dtype=np.int64))
    counts = np.bincount(g.receiver[ids], minlength=g.n_nodes)
    rowptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return rowptr, g.sender[ids], g.evec[ids], ids


def edges_of_receivers(g: Graph, recv):
    """Sub-graph with the in-edges of the given receivers."""
    recv = np.unique(np.asarray(recv))
    ids = (np.concatenate([np.arange(g.rowptr[b], g.rowptr[b + 1]) for b in recv])
           if len(recv) else np.zeros(0, np.int64))
    return subgraph(g, ids)


def edges_of_senders(g: Graph, snd):
    """Sub-graph with the out-edges of the given senders."""
    return subgraph(g, np.nonzero(np.isin(g.sender, np.asarray(snd)))[0])


def random_graph(n_nodes: int, box: float, cutoff: float, seed: int,
                 permute_labels: bool = False) -> Graph:
    """Uniform positions in [0, box)^3 from PCG64(seed); optional random
    relabelling of the nodes (drawn from the same stream, after the positions)."""
    rng = np.random.default_rng(seed)
    pos = rng.uniform(0.0, box, (n_nodes, 3))
    if permute_labels:
        pos = pos[rng.permutation(n_nodes)]
    return radius_graph(pos, cutoff)


# ---------------------------------------------------------------- configs

@dataclass
class ConvProblem:
    name: str
    x_irreps: list
    y_irreps: list
    out_irreps: list
    channels: int
    graph: Graph
    x: np.ndarray   # [N, dx, C] float32 (bf16-exact when bf16)
    w: np.ndarray   # [E, P, C]
    dm: np.ndarray  # [N, dout, C] upstream gradient
    dtype: str = "f32"
    extra: dict = field(default_factory=dict)

    @property
    def n_paths(self):
        return num_paths(self.x_irreps, self.y_irreps, self.out_irreps)


@dataclass
class TPProblem:
    name: str
    x_irreps: list
    y_irreps: list
    out_irreps: list
    channels: int
    x: np.ndarray    # [B, dx, C]
    u: np.ndarray    # [B, 3] random unit vectors (y = harmonics of u)
    w: np.ndarray    # [B, P, C]
    dz: np.ndarray = None  # [B, dout, C] upstream gradient of z
    dtype: str = "f32"


CONV_CONFIGS = {
    "tiny": dict(n=64, box=6.0, cutoff=3.0, x="8x0e+8x1o", lmax=1, out="8x0e+8x1o",
                 weights="normal", dtype="f32", permute=False),
    "water3k": dict(n=3000, density=0.1, cutoff=5.0, x="128x0e+128x1o", lmax=3,
                    out="128x0e+128x1o+128x2e+128x3o", weights="radial_mlp", dtype="f32",
                    permute=False),
    "mace64k": dict(n=64000, density=0.1, cutoff=5.0, x="128x0e+128x1o", lmax=3,
                    out="128x0e+128x1o+128x2e+128x3o", weights="normal", dtype="f32",
                    permute=False),
    # the 64k workload with every parity-allowed output up to l = 3 (13 paths)
    "mace64k_all": dict(n=64000, density=0.1, cutoff=5.0, x="128x0e+128x1o", lmax=3,
                        out="128x0e+128x1o+128x1e+128x2e+128x2o+128x3o+128x3e",
                        weights="normal", dtype="f32", permute=False),
    "ho20k": dict(n=20000, density=0.1, cutoff=5.0, x="64x0e+64x1o+64x2e+64x3o", lmax=3,
                  out="64x0e+64x1o+64x2e+64x3o", weights="normal", dtype="bf16", permute=True),
}

TP_CONFIG = dict(rows=200000, x="128x0e+128x1o+128x2e", lmax=3,
                 out="128x0e+128x1o+128x2e+128x3o", dtype="f32")

# stream tags (one independent stream per drawn array)
TAG_X, TAG_W, TAG_DM, TAG_W1, TAG_W2, TAG_U = 1, 2, 3, 4, 5, 6


def bessel_basis(d: np.ndarray, cutoff: float, n: int = 8) -> np.ndarray:
    """sqrt(2/rc) sin(k pi d / rc) / d, k = 1..n (no envelope), fp64."""
    k = np.arange(1, n + 1, dtype=np.float64)
    d = np.maximum(d.astype(np.float64), 1e-9)[:, None]
    return np.sqrt(2.0 / cutoff) * np.sin(k * np.pi * d / cutoff) / d


def radial_mlp_weights(evec: np.ndarray, cutoff: float, n_paths: int, channels: int,
                       seed: int) -> np.ndarray:
    """Random 2-layer MLP (8 -> 64, SiLU, -> P*C), evaluated in fp64 and
    stored as float32 [E, P, C].  W1 ~ N(0,1)/sqrt(8), W2 ~ N(0,1)/sqrt(64)."""
    W1 = normal((8, 64), seed, TAG_W1).astype(np.float64) / np.sqrt(8.0)
    W2 = normal((64, n_paths * channels), seed, TAG_W2).astype(np.float64) / np.sqrt(64.0)
    E = evec.shape[0]
    out = np.empty((E, n_paths, channels), dtype=np.float32)
    for lo in range(0, E, 1 << 15):
        hi = min(E, lo + (1 << 15))
        d = np.linalg.norm(evec[lo:hi].astype(np.float64), axis=1)
        h = bessel_basis(d, cutoff) @ W1
        h = h / (1.0 + np.exp(-h))  # SiLU
        out[lo:hi] = (h @ W2).reshape(hi - lo, n_paths, channels)
    return out


def make_conv(name: str, seed: int = 0, with_dm: bool = True) -> ConvProblem:
    cfg = CONV_CONFIGS[name]
    n = cfg["n"]
    box = cfg["box"] if "box" in cfg else (n / cfg["density"]) ** (1.0 / 3.0)
    g = random_graph(n, box, cfg["cutoff"], seed, permute_labels=cfg["permute"])
    C, xi = parse_irreps(cfg["x"])
    _, oi = parse_irreps(cfg["out"])
    yi = sh_irreps(cfg["lmax"])
    P = num_paths(xi, yi, oi)
    x = normal((n, dim(xi), C), seed, TAG_X)
    if cfg["weights"] == "radial_mlp":
        w = radial_mlp_weights(g.evec, cfg["cutoff"], P, C, seed)
    else:
        w = normal((g.n_edges, P, C), seed, TAG_W)
    dm = normal((n, dim(oi), C), seed, TAG_DM) if with_dm else None
    if cfg["dtype"] == "bf16":
        x, w = round_bf16(x), round_bf16(w)
        dm = round_bf16(dm) if dm is not None else None
    return ConvProblem(name=name, x_irreps=xi, y_irreps=yi, out_irreps=oi, channels=C, graph=g,
                       x=x, w=w, dm=dm, dtype=cfg["dtype"], extra=dict(cfg, box=box))


def degree_irreps(L: int, skew: bool = False):
    """Every irrep 0..L once: parity (-1)^l, or (-1)^(l+1) when skew."""
    return [(l, (1 if l % 2 == 0 else -1) * (-1 if skew else 1)) for l in range(L + 1)]


def make_conv_degree(L: int, seed: int = 0, n_nodes: int = 2048, channels: int = 128,
                     box: float = 26.75, cutoff: float = 5.0, dtype: str = "f32",
                     with_dm: bool = True) -> ConvProblem:
    """The convolution at degree L: x and out = every irrep 0..L (natural
    parity), y = SH 0..L, N(0,1) node features, weights and cotangent."""
    g = random_graph(n_nodes, box, cutoff, seed)
    xi = oi = degree_irreps(L)
    yi = sh_irreps(L)
    P = num_paths(xi, yi, oi)
    x = normal((n_nodes, dim(xi), channels), seed, TAG_X)
    w = normal((g.n_edges, P, channels), seed, TAG_W)
    dm = normal((n_nodes, dim(oi), channels), seed, TAG_DM) if with_dm else None
    if dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
        dm = round_bf16(dm) if dm is not None else None
    return ConvProblem(name=f"deg{L}", x_irreps=xi, y_irreps=yi, out_irreps=oi,
                       channels=channels, graph=g, x=x, w=w, dm=dm, dtype=dtype,
                       extra=dict(n=n_nodes, box=box, cutoff=cutoff, lmax=L))


def make_tp(seed: int = 0, rows: int | None = None, with_dz: bool = False) -> TPProblem:
    cfg = TP_CONFIG
    B = cfg["rows"] if rows is None else rows
    C, xi = parse_irreps(cfg["x"])
    _, oi = parse_irreps(cfg["out"])
    yi = sh_irreps(cfg["lmax"])
    P = num_paths(xi, yi, oi)
    u = normal((B, 3), seed, TAG_U).astype(np.float64)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    x = normal((B, dim(xi), C), seed, TAG_X)
    w = normal((B, P, C), seed, TAG_W)
    dz = normal((B, dim(oi), C), seed, TAG_DM) if with_dz else None
    return TPProblem(name="tp", x_irreps=xi, y_irreps=yi, out_irreps=oi, channels=C, x=x,
                     u=u.astype(np.float32), w=w, dz=dz, dtype="f32")
