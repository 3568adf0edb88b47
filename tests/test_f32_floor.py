"""The float32 rounding floor of the forward convolution on the water-box
workload (radial-MLP weights that grow as 1/d at the closest pairs, so one
edge dominates the largest outputs), from the float32 emulation of the
kernel's own arithmetic order (tests/f32_emulation.py), against the oracle.

Collapsed outputs (two edge groups per wavefront at C = 128): the floor is
under the fp32 gate of 1e-5.  One output block per path (one edge group of 64
lanes at two channels per lane, so each receiver's edges are summed in one
sequence): the floor is 1.22e-5, above the gate -- the tests of that mode
compare the GPU with this emulation instead (tests/test_gpu_per_path.py)."""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from tests import f32_emulation as F


@pytest.fixture(scope="module")
def water3k():
    return S.make_conv("water3k", with_dm=False)


def _floor(p, per_path, groups):
    m = F.conv_forward_f32(p, per_path, groups)
    od = O.Desc(p.x_irreps, p.y_irreps, p.out_irreps, p.channels, per_path=per_path)
    ref = O.conv_forward(od, p.graph.rowptr, p.graph.sender, p.x, p.w, evec=p.graph.evec)
    return float(np.abs(m - ref).max() / np.sqrt(np.mean(ref ** 2)))


def test_floor_collapsed_water3k(water3k):
    e = _floor(water3k, False, 2)
    assert 8e-6 < e < 1e-5, e


def test_floor_per_path_water3k(water3k):
    e = _floor(water3k, True, 1)
    assert 1.1e-5 < e < 1.35e-5, e
