"""GPU parity of the per-irrep channel mixing (e3j A.3 Eq.5) on the fp32
matrix cores, through the C ABI, against the fp64 oracle.

Tolerance: max|gpu - oracle| / RMS(oracle) <= 1e-5 per output (fp32
storage); bf16 storage: 2e-2 ahead of the output's own rounding.  Row counts
are chosen ragged against the 32-row MFMA tiles.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_amd import synth as S
from oracle import oracle as O
from tests.gpu_util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from clebsch_gordan_tensor_amd import api
    api.lib()
    return api


def _ir(s):
    return S.parse_irreps(s)[1]


def _case(ins, outs, rows, cin, cout, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, S.dim(ins), cin)).astype(np.float32)
    W = (rng.standard_normal((O.linear_num_weights(ins, outs), cin, cout)) /
         np.sqrt(cin)).astype(np.float32)
    return x, W


@pytest.mark.parametrize("xs,os_,rows,cin,cout", [
    ("0e+1o+2e+3o", "0e+1o+2e+3o", 3001, 128, 128),   # the 64k config's features
    ("0e+1o", "0e+1o+2e+3o", 1111, 128, 128),         # unmatched output blocks are zero
    ("0e+0e+1o", "0e+1o", 777, 64, 32),               # two input blocks of one type
    ("0e+1o+1e", "1e+0e+1o", 555, 8, 256),            # two column slabs
    ("0e+2e", "2e+0e", 333, 32, 96),                  # a 96-column slab
    ("3o", "3o", 1, 128, 128),                        # a single row
])
def test_linear_matches_oracle(gpu, xs, os_, rows, cin, cout):
    ins, outs = _ir(xs), _ir(os_)
    x, W = _case(ins, outs, rows, cin, cout, 90 + rows)
    y = host(gpu.linear(ins, outs, dev(x), dev(W)))
    ref = O.linear(ins, outs, x, W)
    assert_close(y, ref, TOL_F32, f"linear {xs}->{os_}")
    if os_ == "0e+1o+2e+3o" and xs == "0e+1o":
        assert np.all(y[:, 4:] == 0.0)


def test_linear_bf16_storage(gpu):
    ins = outs = _ir("0e+1o+2e+3o")
    x, W = _case(ins, outs, 1500, 128, 128, 95)
    x = S.round_bf16(x)
    y = host(gpu.linear(ins, outs, dev(x, "bf16"), dev(W)))
    assert_close(y, O.linear(ins, outs, x, W), TOL_BF16, "linear bf16", bf16_out=True)


def test_linear_full_size_sampled(gpu):
    # the node features of the 64k-atom workload
    ins = outs = _ir("0e+1o+2e+3o")
    x, W = _case(ins, outs, 64000, 128, 128, 96)
    y = gpu.linear(ins, outs, dev(x), dev(W))
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(1).choice(64000, 1500, replace=False))
    ref = O.linear(ins, outs, x[idx], W)
    assert_close(host(y[torch.from_numpy(idx).cuda()]), ref, TOL_F32, "linear 64k")


def test_linear_deterministic_and_empty(gpu):
    ins = outs = _ir("0e+1o")
    x, W = _case(ins, outs, 999, 64, 64, 97)
    a = gpu.linear(ins, outs, dev(x), dev(W))
    b = gpu.linear(ins, outs, dev(x), dev(W))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    e = gpu.linear(ins, outs, torch.empty((0, 4, 64), device="cuda"), dev(W))
    torch.cuda.synchronize()
    assert e.shape == (0, 4, 64)
