"""Helpers shared by the GPU tests: device upload, sub-graph slicing for
sampled oracle checks, and the tolerance metric max|gpu - ref| / RMS(ref)."""
from __future__ import annotations

import numpy as np

from clebsch_gordan_tensor_amd import synth as S

TOL_F32 = 1e-5   # max abs error / RMS of the oracle output, fp32 storage
TOL_BF16 = 2e-2  # bf16 storage, fp32 accumulation


def dev(a, dtype="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def host(t):
    import torch
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    err = np.abs(got - ref).max()
    return float(err / rms) if rms > 0 else float(err)


BF16_HALF_ULP = 2.0 ** -8  # round-to-nearest error of a bf16 value, relative to it


def rel_err_bf16(got, ref):
    """Error of a bf16-stored output ahead of its own storage rounding:
    max(|got - ref| - 2^-8 max(|got|, |ref|), 0) / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.abs(got - ref) - BF16_HALF_ULP * np.maximum(np.abs(got), np.abs(ref))
    e = float(np.maximum(excess, 0.0).max())
    return e / rms if rms > 0 else e


def assert_close(got, ref, tol, what="", bf16_out=False):
    if bf16_out:
        e = rel_err_bf16(got, ref)
    else:
        e = rel_err(got, ref)
    print(f"[err] {what}: {e:.3e} (gate {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max|err|/rms = {e:.3e} > {tol:.1e}"
    return e


edges_of_receivers = S.edges_of_receivers
edges_of_senders = S.edges_of_senders
subgraph = S.subgraph
