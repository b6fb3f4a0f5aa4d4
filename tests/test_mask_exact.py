"""Bit-exact properties of the HIP path: masked keys contribute exactly 0,
keys past N are never read, nothing is written past O / LSE, and repeated
runs agree bit for bit."""

import math

import pytest
import torch

import io_aware_exact_fa1_amd as fa
import workloads
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _call(q, k, v, o, lse, causal, scale):
    B, H, N, d = q.shape
    f = fa.fa_fwd if q.dtype == torch.bfloat16 else fa.fa_fwd_f32
    st = f(q, k, v, o, lse, B, H, N, d, scale, causal)
    assert st == fa.FA_OK, fa.fa_strerror(st)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_future_keys_contribute_exactly_zero(dtype, d):
    N = 300
    q, k, v = (x.cuda() for x in workloads.make_qkv(1, 2, N, d, dtype, seed=21))
    o0, l0 = fa.forward(q, k, v, causal=True)
    for r in (1, 37, 64, 128, 129, 250):
        say("future keys", dtype, d, r)
        k2, v2 = k.clone(), v.clone()
        g = torch.Generator(device="cpu").manual_seed(r)
        k2[:, :, r:] = (torch.randn(k2[:, :, r:].shape, generator=g) * 1e4).to(dtype).cuda()
        v2[:, :, r:] = (-torch.randn(v2[:, :, r:].shape, generator=g) * 1e4).to(dtype).cuda()
        o1, l1 = fa.forward(q, k2, v2, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, :, :r], o0[:, :, :r]), r
        assert torch.equal(l1[:, :, :r], l0[:, :, :r]), r


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 45, 100, 257])
@pytest.mark.parametrize("causal", [False, True])
def test_tail_keys_never_read_and_no_stray_writes(dtype, d, N, causal):
    """Q, K, V sit at the start of NaN-filled buffers; O and LSE at the start
    of sentinel-filled buffers.  Results must be finite, equal bit for bit to
    a run on exact-size buffers, and the sentinels must survive."""
    say("guard band", dtype, d, N, causal)
    q, k, v = (x.cuda() for x in workloads.make_qkv(1, 1, N, d, dtype, seed=31 + N))
    n = N * d
    pad = 4096
    bufs = []
    for x in (q, k, v):
        b = torch.full((n + pad,), float("nan"), dtype=dtype, device="cuda")
        b[:n] = x.reshape(-1)
        bufs.append(b)
    ob = torch.full((n + pad,), 7.0, dtype=dtype, device="cuda")
    lb = torch.full((N + pad,), -3.0, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    f = fa.fa_fwd if dtype == torch.bfloat16 else fa.fa_fwd_f32
    st = f(bufs[0], bufs[1], bufs[2], ob, lb, 1, 1, N, d, scale, causal)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    o_ref, l_ref = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(ob[:n]).all() and torch.isfinite(lb[:N]).all()
    assert torch.equal(ob[:n], o_ref.reshape(-1)) and torch.equal(lb[:N], l_ref.reshape(-1))
    assert bool((ob[n:] == 7.0).all()) and bool((lb[N:] == -3.0).all())


@pytest.mark.parametrize("name", ["ragged_n1000_d64_causal", "n4096_d128_causal"])
def test_deterministic(name):
    w = workloads.get(name)
    q, k, v = (x.cuda() for x in workloads.make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, w.k_mult))
    say("determinism", name)
    o1, l1 = fa.forward(q, k, v, causal=w.causal)
    o2, l2 = fa.forward(q, k, v, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
