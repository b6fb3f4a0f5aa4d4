"""Backward pass on the GPU (through the C ABI) against the fp64 oracle.

The GPU path is the real pipeline: ``fa_fwd`` writes O and LSE, then
``fa_bwd`` recomputes the gradients from them.  The oracle computes the
exact gradients of the same bf16 inputs from the definition
(``attention_bwd_ref``) or, for large shapes, for sampled rows and columns.

Tolerance (bf16 inputs, fp32 accumulation, bf16 outputs), per gradient G
with reference R, measured against the tensor's own scale
``s = max(1, max|R|)`` (absolute for gradients below 1, as for the forward
with N(0,1) inputs): max|G - R| <= BWD_MAX * s and mean|G - R| <= BWD_MEAN * s.
The kernel rounds P and dS to bf16 for the second matrix products (unit
roundoff u = 2^-8 each: bf16 keeps 8 significant bits, so one ulp at 1.0 is
2^-7), rounds the result to bf16 (u again), and takes O and LSE from the
bf16 forward (O rounded to bf16 enters D = O . dO); with cancellation in the
sums over keys of dS (its rows sum to zero) an error of a few units of
roundoff of the largest term is what remains.
"""

import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu, say
from oracle import attention_bwd_cols_ref, attention_bwd_ref, attention_bwd_rows_ref
import io_aware_exact_fa1_amd as fa
import workloads

pytestmark = pytest.mark.gpu

BWD_MAX = 1.6e-2   # max abs error / max |ref|   (about 4 u = 4 * 2^-8, i.e. 2 bf16 ulps at 1.0)
BWD_MEAN = 2.0e-3  # mean abs error / max |ref|


def _inputs(B, H, N, d, causal, seed):
    q, k, v = workloads.make_qkv(B, H, N, d, torch.bfloat16, seed)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed + 7919)
    do = torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do


def _run(q, k, v, do, causal, scale=None):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.float().cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy(), \
        delta.cpu().numpy(), o.float().cpu().numpy()


def _check(name, got, ref, tag):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1.0)
    emax = float(np.max(np.abs(got - ref))) / scale
    emean = float(np.mean(np.abs(got - ref))) / scale
    say(f"{tag} {name}: scale {scale:.3e} max err/scale {emax:.2e} mean err/scale {emean:.2e}")
    assert np.all(np.isfinite(got)), f"{tag} {name}: non-finite output"
    assert emax <= BWD_MAX, f"{tag} {name}: max err {emax:.3e} > {BWD_MAX}"
    assert emean <= BWD_MEAN, f"{tag} {name}: mean err {emean:.3e} > {BWD_MEAN}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 64, 100, 129, 257, 300])
def test_bwd_small_shapes(N, d, causal):
    require_gpu()
    B, H = 1, 2
    q, k, v, do = _inputs(B, H, N, d, causal, seed=1000 + N + d)
    scale = 1.0 / np.sqrt(d)
    tag = f"N={N} d={d} causal={causal}"
    say(f"[bwd] {tag}")
    dq, dk, dv, delta, o = _run(q, k, v, do, causal)
    q, k, v, do = (f64(x) for x in (q, k, v, do))
    for b in range(B):
        for h in range(H):
            rq, rk, rv, rd = attention_bwd_ref(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
            _check("dQ", dq[b, h], rq, tag)
            _check("dK", dk[b, h], rk, tag)
            _check("dV", dv[b, h], rv, tag)
            # D = O . dO with the forward's bf16 O (the workspace is an output too)
            np.testing.assert_allclose(delta[b, h], np.sum(o[b, h] * do[b, h], axis=1),
                                       rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_n1000(causal):
    """B=4, H=16, N=1000, d=64 (the ragged workload's shape), every head."""
    require_gpu()
    w = workloads.get("ragged_n1000_d64_causal" if causal else "ragged_n1000_d64_noncausal")
    q, k, v, do = _inputs(w.B, w.H, w.N, w.d, causal, seed=w.seed)
    tag = f"{w.name}"
    say(f"[bwd] {tag}")
    dq, dk, dv, _, _ = _run(q, k, v, do, causal)
    q, k, v, do = (f64(x) for x in (q, k, v, do))
    for b in range(w.B):
        for h in range(0, w.H, 5):
            rq, rk, rv, _ = attention_bwd_ref(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, causal)
            _check("dQ", dq[b, h], rq, f"{tag} b={b} h={h}")
            _check("dK", dk[b, h], rk, f"{tag} b={b} h={h}")
            _check("dV", dv[b, h], rv, f"{tag} b={b} h={h}")


@pytest.mark.parametrize("name", ["n4096_d128_causal", "n8192_d64_peaky", "longctx_n16384_d128_causal"])
def test_bwd_large_sampled(name):
    """Full-size workloads: dQ on sampled rows, dK and dV on sampled keys,
    of two sampled heads."""
    require_gpu()
    w = workloads.get(name)
    q, k, v = workloads.make_qkv(w.B, w.H, w.N, w.d, torch.bfloat16, w.seed, w.k_mult)
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 7919)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    say(f"[bwd] {name}")
    dq, dk, dv, _, _ = _run(q, k, v, do, w.causal)
    heads = workloads.sample_heads(w.B, w.H, 2, w.seed)
    q, k, v, do = (f64(x[[b for b, _ in heads], [h for _, h in heads]]) for x in (q, k, v, do))
    rows = workloads.sample_rows(w.N, 64, w.seed)
    for i, (b, h) in enumerate(heads):
        rq = attention_bwd_rows_ref(q[i], k[i], v[i], do[i], w.scale, w.causal, rows)
        rk, rv = attention_bwd_cols_ref(q[i], k[i], v[i], do[i], w.scale, w.causal, rows)
        tag = f"{name} b={b} h={h}"
        _check("dQ rows", dq[b, h][rows], rq, tag)
        _check("dK rows", dk[b, h][rows], rk, tag)
        _check("dV rows", dv[b, h][rows], rv, tag)


def test_bwd_causal_future_rows_do_not_touch_dq():
    """Causal: dQ of rows < r depends only on keys/values < r, bitwise."""
    require_gpu()
    N, d = 300, 128
    q, k, v, do = _inputs(1, 2, N, d, True, seed=77)
    dq1 = _run(q, k, v, do, True)[0]
    for r in (1, 64, 129, 255):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, r:] = (torch.randn_like(k2[:, :, r:].float()) * 50).to(torch.bfloat16)
        v2[:, :, r:] = -v2[:, :, r:]
        dq2 = _run(q, k2, v2, do, True)[0]
        assert np.array_equal(dq1[:, :, :r], dq2[:, :, :r]), r


def test_bwd_deterministic():
    require_gpu()
    q, k, v, do = _inputs(2, 3, 513, 64, True, seed=5)
    a = _run(q, k, v, do, True)
    b = _run(q, k, v, do, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_key_shift_and_value_sums():
    """sum over keys of dK ~ 0 and of dV = sum over queries of dO."""
    require_gpu()
    q, k, v, do = _inputs(1, 2, 700, 128, False, seed=9)
    dq, dk, dv, _, _ = _run(q, k, v, do, False)
    do = f64(do)
    for h in range(2):
        ref_dv_sum = do[0, h].sum(axis=0)
        tot = np.abs(dv[0, h]).sum(axis=0).max()
        assert np.max(np.abs(dv[0, h].sum(axis=0) - ref_dv_sum)) <= 2e-2 * tot
        assert np.max(np.abs(dk[0, h].sum(axis=0))) <= 2e-2 * np.abs(dk[0, h]).sum(axis=0).max()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.3])
def test_bwd_scale_variants(scale, d, causal):
    """Negative scale (the kernels flip the sign of Q or K and run with
    |scale|), zero scale (uniform weights) and a larger one; ragged N so that
    diagonal and tail tiles are masked."""
    require_gpu()
    N = 200
    q, k, v, do = _inputs(1, 2, N, d, causal, seed=int(1000 * scale) + d + 31)
    tag = f"scale={scale} d={d} causal={causal}"
    say(f"[bwd] {tag}")
    dq, dk, dv, _, _ = _run(q, k, v, do, causal, scale=scale)
    q, k, v, do = (f64(x) for x in (q, k, v, do))
    for h in range(2):
        rq, rk, rv, _ = attention_bwd_ref(q[0, h], k[0, h], v[0, h], do[0, h], scale, causal)
        _check("dQ", dq[0, h], rq, f"{tag} h={h}")
        _check("dK", dk[0, h], rk, f"{tag} h={h}")
        _check("dV", dv[0, h], rv, f"{tag} h={h}")


def test_bwd_many_heads_short_rows():
    """B = 8, H = 32, N = 129 (causal): 256 heads of two key tiles (one of a
    single row); every 17th head against the oracle."""
    require_gpu()
    q, k, v, do = _inputs(8, 32, 129, 128, True, seed=4242)
    say("[bwd] many heads")
    dq, dk, dv, _, _ = _run(q, k, v, do, True)
    q, k, v, do = (f64(x) for x in (q, k, v, do))
    scale = 1.0 / np.sqrt(128)
    for idx in range(0, 8 * 32, 17):
        b, h = divmod(idx, 32)
        rq, rk, rv, _ = attention_bwd_ref(q[b, h], k[b, h], v[b, h], do[b, h], scale, True)
        _check("dQ", dq[b, h], rq, f"b={b} h={h}")
        _check("dK", dk[b, h], rk, f"b={b} h={h}")
        _check("dV", dv[b, h], rv, f"b={b} h={h}")
