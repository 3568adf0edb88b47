"""GPU test of e3_conv_backward_noalloc (the backward for callers that cannot
allocate device memory: its per-graph index is built inside the call in the
library's fixed device scratch) through the C ABI, against e3_conv_backward
with a workspace prepared by e3_conv_prepare_transpose: two calls in a row,
the second on a smaller graph (the scratch keeps the first call's contents),
then the first graph again; results bitwise equal.  Also: a graph with
padding edges, and the size limit rejected before any launch."""
import ctypes as C

import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _case(g, C, seed, dtype="f32"):
    from clebsch_gordan_tensor_amd import api
    xi, yi, oi = [(0, 1), (1, -1)], S.sh_irreps(3), [(0, 1), (1, -1), (2, 1), (3, -1)]
    d = api.Desc(xi, yi, oi, C)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((g.n_nodes, 4, C)).astype(np.float32)
    w = rng.standard_normal((g.n_edges, api.num_paths(d), C)).astype(np.float32)
    dm = rng.standard_normal((g.n_nodes, 16, C)).astype(np.float32)
    return d, dev(g.rowptr), dev(g.sender), dev(g.evec), dev(x, dtype), dev(w, dtype), dev(dm, dtype)


def _same(a, b):
    bits = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(bits), b.view(bits))


def _both(gpu, d, rowptr, sender, ev, x, w, dm):
    ws = gpu.conv_prepare_transpose(rowptr, sender, edge_vec=ev)
    ref = gpu.conv_backward(d, rowptr, sender, ws, ev, x, w, dm)
    got = gpu.conv_backward_noalloc(d, rowptr, sender, ev, x, w, dm)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_prepared_backward_twice(gpu):
    big = S.make_conv("water3k", with_dm=False).graph          # 3,000 nodes, 130,158 edges
    small = S.random_graph(700, 19.0, 5.0, 21)                  # a smaller graph afterwards
    for g, C, seed in ((big, 128, 1), (small, 64, 2), (big, 128, 1)):
        ref, got = _both(gpu, *_case(g, C, seed))
        for name, a, b in zip(("dx", "dw", "dY"), ref, got):
            assert _same(a, b), f"{g.n_nodes} nodes: {name} differs"


def test_noalloc_padding_and_bf16(gpu):
    from tests.test_oracle_conv import with_padding
    g = with_padding(S.random_graph(500, 17.0, 5.0, 23), 9, 23)
    ref, got = _both(gpu, *_case(g, 64, 3, "bf16"))
    for name, a, b in zip(("dx", "dw", "dY"), ref, got):
        assert _same(a, b), f"padded bf16: {name} differs"
    pad = np.flatnonzero(g.sender < 0)
    assert pad.size and torch.all(got[1][dev(pad).long()] == 0)


def test_noalloc_rejects_graphs_past_its_limit(gpu):
    from clebsch_gordan_tensor_amd import api
    d = api.Desc([(0, 1), (1, -1)], S.sh_irreps(3), [(0, 1), (1, -1), (2, 1), (3, -1)], 64)
    L = api.lib()
    for n, e in ((1 << 17, (1 << 22) + 1), ((1 << 17) + 1, 10)):
        st = L.e3_conv_backward_noalloc(C.byref(d.c()), n, e, None, None, None, None, None, None,
                                        None, None, None, api.E3_F32, None)
        assert st == -3, st  # E3_ERR_UNSUPPORTED, before any pointer is used
        assert b"at most" in L.e3_last_error()
