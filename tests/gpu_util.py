"""Shared helpers of the GPU parity tests (HIP path vs the fp64 oracle)."""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_fa1_amd as fa

# Tolerances of the attention forward against the fp64 oracle:
#   fp32 inputs: max |dO| <= 1e-5, max |dLSE| <= 1e-5;
#   bf16 inputs (fp32 accumulation): max |dO| <= 2e-2, mean |dO| <= 2e-3,
#   max |dLSE| <= 1e-3.
TOL = {
    torch.float32: dict(o_max=1e-5, o_mean=None, lse_max=1e-5),
    torch.bfloat16: dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3),
}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    fa.load_library()


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(q, k, v, causal, scale):
    """q, k, v CPU tensors -> (O, LSE) CUDA tensors from the HIP library."""
    qd, kd, vd = (x.to("cuda") for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    do = np.abs(np.asarray(o_gpu, np.float64) - o_ref)
    dl = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
    return float(do.max()), float(do.mean()), float(dl.max())


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what="", tol=None):
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what
    tol = TOL[dtype] if tol is None else tol
    omax, omean, lmax = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    say(f"{what}: max|dO|={omax:.3e} mean|dO|={omean:.3e} max|dLSE|={lmax:.3e}")
    assert omax <= tol["o_max"], (what, omax)
    if tol["o_mean"] is not None:
        assert omean <= tol["o_mean"], (what, omean)
    assert lmax <= tol["lse_max"], (what, lmax)
    return omax, omean, lmax
