"""GPU parity of the signature with every parity-allowed output up to l = 3,
pseudotensors included (x 128x(0e+1o), Y l <= 3, out
0e+1o+1e+2e+2o+3o+3e, 13 paths): the other reading of the 64k workload's
"output lmax=3 all paths".  Gates as for the collapsed convolution."""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from tests.gpu_util import TOL_F32, assert_close, dev, host
from tests.test_gpu_parity import _full_conv_check, desc_pair, oracle_all, run_conv

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ALL = S.parse_irreps("128x0e+128x1o+128x1e+128x2e+128x2o+128x3o+128x3e")[1]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _water3k_all():
    p = S.make_conv("water3k", with_dm=False)
    rng = np.random.default_rng(150)
    P = S.num_paths(p.x_irreps, p.y_irreps, ALL)
    assert P == 13 and S.dim(ALL) == 31
    w = rng.standard_normal((p.graph.n_edges, P, 128)).astype(np.float32)
    dm = rng.standard_normal((p.graph.n_nodes, 31, 128)).astype(np.float32)
    return p, w, dm


def test_all_outputs_water3k_full(gpu):
    p, w, dm = _water3k_all()
    d, od = desc_pair(p.x_irreps, p.y_irreps, ALL, 128)
    got = run_conv(gpu, d, p.graph, p.x, w, dm)
    ref = oracle_all(od, p.graph, p.x, w, dm)
    for k, a, b in zip(("m", "dx", "dw", "dY"), got, ref):
        assert_close(a, b, TOL_F32, f"all-outputs water3k:{k}")


def test_all_outputs_inversion_parity(gpu):
    # pos -> -pos flips every edge vector; x^(l,p) -> p x  =>  m^(L,p) -> p m,
    # which separates the pseudotensor blocks from the tensor blocks
    p, w, _ = _water3k_all()
    g = p.graph
    d, _ = desc_pair(p.x_irreps, p.y_irreps, ALL, 128)
    sx = np.concatenate([[q] * (2 * l + 1) for l, q in p.x_irreps])[None, :, None]
    so = np.concatenate([[q] * (2 * l + 1) for l, q in ALL])[None, :, None]
    rowptr, sender = dev(g.rowptr), dev(g.sender)
    m = host(gpu.conv_forward(d, rowptr, sender, dev(g.evec), dev(p.x), dev(w)))
    mi = host(gpu.conv_forward(d, rowptr, sender, dev(-g.evec), dev((sx * p.x).astype(np.float32)),
                               dev(w)))
    assert_close(mi, so * m, TOL_F32, "inversion")


@pytest.mark.timeout(900)
def test_all_outputs_mace64k_full(gpu):
    _full_conv_check(gpu, S.make_conv("mace64k_all"), TOL_F32)
