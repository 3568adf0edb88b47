"""Write tests/golden/tiny_conv_sample.json from the oracle alone.

The fixture is a regression guard: a few outputs of the tiny configuration
(64 nodes in a 6 A cube, 3 A cutoff, seed 0, 8x(0e+1o) with harmonics up to
l = 1) computed by the fp64 oracle.  Any later change to the oracle's
arithmetic must reproduce these numbers or say why in its commit.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from clebsch_gordan_tensor_amd import synth as S  # noqa: E402
from oracle import oracle as O  # noqa: E402

RECV = [0, 17, 63]
EDGES = [0, 511, 1023]


def compute():
    p = S.make_conv("tiny")
    g = p.graph
    d = O.Desc(p.x_irreps, p.y_irreps, p.out_irreps, p.channels)
    m = O.conv_forward(d, g.rowptr, g.sender, p.x, p.w, evec=g.evec, rows=RECV)
    dx = O.conv_backward_dx(d, g.rowptr, g.sender, p.w, p.dm, evec=g.evec, rows=RECV)
    dw, dY = O.conv_backward_edge(d, g.rowptr, g.sender, p.x, p.w, p.dm, evec=g.evec,
                                  edges=EDGES)
    return dict(n_edges=g.n_edges, receivers=RECV, edges=EDGES, m=m.tolist(), dx=dx.tolist(),
                dw=dw.tolist(), dY=dY.tolist())


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_conv_sample.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=0)
    print(out)
