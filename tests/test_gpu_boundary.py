"""GPU checks of the boundary's graph handling through the C ABI: the debug
graph check (E3_CHECK flag and e3_check_graph) on device arrays, and the
per-graph preparation (device-side traversal with a fixed number of level
launches) on graphs deeper than those launches, with several components and
isolated nodes, checked through the convolution against the fp64 oracle."""
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


def _problem(g, C=16, seed=0):
    from clebsch_gordan_tensor_amd import api
    xi, yi, oi = [(0, 1), (1, -1)], S.sh_irreps(3), [(0, 1), (1, -1), (2, 1), (3, -1)]
    d = api.Desc(xi, yi, oi, C)
    od = O.Desc(xi, yi, oi, C)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((g.n_nodes, 4, C)).astype(np.float32)
    w = rng.standard_normal((g.n_edges, api.num_paths(d), C)).astype(np.float32)
    dm = rng.standard_normal((g.n_nodes, 16, C)).astype(np.float32)
    return d, od, x, w, dm


def _graph_from_pairs(pos, snd, rcv):
    snd, rcv = np.asarray(snd, np.int64), np.asarray(rcv, np.int64)
    order = np.lexsort((snd, rcv))
    snd, rcv = snd[order], rcv[order]
    n = pos.shape[0]
    rowptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(rcv, minlength=n), out=rowptr[1:])
    return S.Graph(pos=pos, rowptr=rowptr.astype(np.int32), sender=snd.astype(np.int32),
                   receiver=rcv.astype(np.int32), evec=(pos[rcv] - pos[snd]).astype(np.float32))


def _conv_vs_oracle(gpu, g, what, seed=0):
    d, od, x, w, dm = _problem(g, seed=seed)
    rowptr, sender, ev = dev(g.rowptr), dev(g.sender), dev(g.evec)
    ws = gpu.conv_prepare_transpose(rowptr, sender, edge_vec=ev)
    m = gpu.conv_forward(d, rowptr, sender, ev, dev(x), dev(w), workspace=ws)
    dx, dw, dY = gpu.conv_backward(d, rowptr, sender, ws, ev, dev(x), dev(w), dev(dm))
    torch.cuda.synchronize()
    ref = (O.conv_forward(od, g.rowptr, g.sender, x, w, evec=g.evec),
           O.conv_backward_dx(od, g.rowptr, g.sender, w, dm, evec=g.evec),
           *O.conv_backward_edge(od, g.rowptr, g.sender, x, w, dm, evec=g.evec))
    for k, a, b in zip(("m", "dx", "dw", "dY"), (m, dx, dw, dY), ref):
        assert_close(host(a), b, TOL_F32, f"{what}:{k}")


def test_prepare_chain_deeper_than_traversal_launches(gpu):
    # a path of 300 nodes 2 A apart (cutoff 2.5 A): 299 traversal levels
    # from node 0, far more than the fixed launches; the nodes the traversal
    # does not reach are appended, and every node is still handled once
    n = 300
    pos = np.zeros((n, 3))
    pos[:, 0] = 2.0 * np.arange(n)
    pos[:, 1] = 0.3 * np.sin(np.arange(n))
    i = np.arange(n - 1)
    g = _graph_from_pairs(pos, np.concatenate([i, i + 1]), np.concatenate([i + 1, i]))
    _conv_vs_oracle(gpu, g, "chain")


def test_prepare_components_and_isolated_nodes(gpu):
    # three clusters far apart, plus isolated nodes (no edges at all)
    rng = np.random.default_rng(31)
    parts = [rng.uniform(0, 6, (60, 3)) + off for off in ([0, 0, 0], [100, 0, 0], [0, 100, 0])]
    pos = np.concatenate(parts + [np.array([[50.0, 50, 50], [-50, -50, -50]])])
    g = S.radius_graph(pos[rng.permutation(pos.shape[0])], 3.0)
    assert np.sum(np.diff(g.rowptr) == 0) >= 2
    _conv_vs_oracle(gpu, g, "components", seed=1)


def test_check_flag_rejects_malformed_graph(gpu):
    from clebsch_gordan_tensor_amd import api
    g = S.make_conv("tiny", with_dm=False).graph
    d, od, x, w, dm = _problem(g, seed=2)
    dc = d.with_flags(d.flags | api.E3_CHECK)
    rowptr, sender, ev = dev(g.rowptr), dev(g.sender), dev(g.evec)
    ws = gpu.conv_prepare_transpose(rowptr, sender, edge_vec=ev)
    m = gpu.conv_forward(d, rowptr, sender, ev, dev(x), dev(w), workspace=ws)
    mc = gpu.conv_forward(dc, rowptr, sender, ev, dev(x), dev(w), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(m.view(torch.int32), mc.view(torch.int32))
    gpu.check_graph(rowptr, sender)
    bad_sender = g.sender.copy()
    bad_sender[11] = g.n_nodes + 5
    bad_rowptr = g.rowptr.copy()
    bad_rowptr[7] = bad_rowptr[8] + 1
    for rp, sn, what in ((g.rowptr, bad_sender, "sender["), (bad_rowptr, g.sender, "decreases")):
        out = torch.full((g.n_nodes, 16, 16), 7.0, device="cuda")
        with pytest.raises(api.E3Error) as ei:
            gpu.conv_forward(dc, dev(rp), dev(sn), ev, dev(x), dev(w), out=out)
        assert ei.value.status == api.E3_ERR_GRAPH and what in str(ei.value)
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)  # nothing was launched
        with pytest.raises(api.E3Error) as ei:
            gpu.conv_backward(dc, dev(rp), dev(sn), ws, ev, dev(x), dev(w), dev(dm))
        assert ei.value.status == api.E3_ERR_GRAPH
        with pytest.raises(api.E3Error) as ei:
            gpu.check_graph(dev(rp), dev(sn))
        assert ei.value.status == api.E3_ERR_GRAPH
