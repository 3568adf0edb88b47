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


# ----------------------------------------------------------------- backward

def _bwd_case(ins, outs, rows, cin, cout, seed):
    x, W = _case(ins, outs, rows, cin, cout, seed)
    dy = np.random.default_rng(seed + 1).standard_normal(
        (rows, S.dim(outs), cout)).astype(np.float32)
    return x, W, dy


@pytest.mark.parametrize("xs,os_,rows,cin,cout", [
    ("0e+1o+2e+3o", "0e+1o+2e+3o", 3001, 128, 128),
    ("0e+1o", "0e+1o+2e+3o", 1111, 128, 128),     # output blocks without a source
    ("0e+0e+1o+2e", "0e+1o", 777, 64, 32),        # an input block without a target
    ("1o+0e", "0e+1o+1o", 555, 32, 256),          # two targets of one input block
])
def test_linear_backward_matches_oracle(gpu, xs, os_, rows, cin, cout):
    ins, outs = _ir(xs), _ir(os_)
    x, W, dy = _bwd_case(ins, outs, rows, cin, cout, 110 + rows)
    dx, dW = gpu.linear_backward(ins, outs, dev(x), dev(W), dev(dy))
    rdx, rdW = O.linear_backward(ins, outs, x, W, dy)
    assert_close(host(dx), rdx, TOL_F32, f"linear dx {xs}->{os_}")
    assert_close(host(dW), rdW, TOL_F32, f"linear dW {xs}->{os_}")


def test_linear_backward_bf16(gpu):
    ins = outs = _ir("0e+1o+2e+3o")
    x, W, dy = _bwd_case(ins, outs, 1500, 128, 128, 120)
    x, dy = S.round_bf16(x), S.round_bf16(dy)
    dx, dW = gpu.linear_backward(ins, outs, dev(x, "bf16"), dev(W), dev(dy, "bf16"))
    rdx, rdW = O.linear_backward(ins, outs, x, W, dy)
    assert_close(host(dx), rdx, TOL_BF16, "linear dx bf16", bf16_out=True)
    assert_close(host(dW), rdW, TOL_F32, "linear dW bf16 inputs")  # dW is float32


def test_linear_backward_full_size(gpu):
    # 64k rows: dx and dW (a sum over all 64,000 x 16 rows) element-wise
    # against the oracle; and the bilinear identity <dW, W> = <dx, x> =
    # <dy, y> (y from the forward)
    ins = outs = _ir("0e+1o+2e+3o")
    x, W, dy = _bwd_case(ins, outs, 64000, 128, 128, 121)
    xd, Wd, dyd = dev(x), dev(W), dev(dy)
    dx, dW = gpu.linear_backward(ins, outs, xd, Wd, dyd)
    y = gpu.linear(ins, outs, xd, Wd)
    torch.cuda.synchronize()
    rdx, rdW = O.linear_backward(ins, outs, x, W, dy)
    assert_close(host(dx), rdx, TOL_F32, "linear dx 64k")
    assert_close(host(dW), rdW, TOL_F32, "linear dW 64k")
    f64 = lambda t: host(t).astype(np.float64)
    ref = np.vdot(dy.astype(np.float64), f64(y))
    for v in (np.vdot(f64(dW), W.astype(np.float64)), np.vdot(f64(dx), x.astype(np.float64))):
        assert abs(v - ref) <= 1e-5 * abs(ref)


def test_linear_backward_no_rows_gives_zero_dW(gpu):
    ins = outs = _ir("0e+1o")
    W = dev(np.ones((2, 32, 32), np.float32))
    dW = torch.full((2, 32, 32), 7.0, device="cuda")
    gpu.linear_backward(ins, outs, torch.empty((0, 4, 32), device="cuda"), W,
                        torch.empty((0, 4, 32), device="cuda"), dW=dW)
    torch.cuda.synchronize()
    assert torch.all(dW == 0)


def test_linear_backward_deterministic(gpu):
    ins = outs = _ir("0e+1o+2e")
    x, W, dy = _bwd_case(ins, outs, 5000, 64, 64, 122)
    a = gpu.linear_backward(ins, outs, dev(x), dev(W), dev(dy))
    b = gpu.linear_backward(ins, outs, dev(x), dev(W), dev(dy))
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))


@pytest.mark.parametrize("cin,cout", [(64, 96), (256, 160), (128, 32)])
def test_linear_bf16_matrix_core_shapes(gpu, cin, cout):
    # bf16 storage runs on the bf16 matrix cores for Cin in {64, 128, 256}
    # (W rounded to bf16 in the kernel); any Cout that is a multiple of 32
    ins = outs = _ir("0e+1o+2e")
    x, W = _case(ins, outs, 700, cin, cout, 130 + cin)
    x = S.round_bf16(x)
    y = host(gpu.linear(ins, outs, dev(x, "bf16"), dev(W)))
    assert_close(y, O.linear(ins, outs, x, W), TOL_BF16, f"linear bf16 {cin}->{cout}",
                 bf16_out=True)


@pytest.mark.parametrize("cin,cout", [(64, 64), (128, 256)])
def test_linear_backward_bf16_matrix_core_shapes(gpu, cin, cout):
    # dx = dy W^T: the bf16 matrix-core path with Cout as the contraction
    ins = outs = _ir("0e+1o")
    x, W, dy = _bwd_case(ins, outs, 600, cin, cout, 140 + cout)
    x, dy = S.round_bf16(x), S.round_bf16(dy)
    dx, dW = gpu.linear_backward(ins, outs, dev(x, "bf16"), dev(W), dev(dy, "bf16"))
    rdx, rdW = O.linear_backward(ins, outs, x, W, dy)
    assert_close(host(dx), rdx, TOL_BF16, f"linear dx bf16 {cin}->{cout}", bf16_out=True)
    assert_close(host(dW), rdW, TOL_F32, f"linear dW bf16 inputs {cin}->{cout}")
