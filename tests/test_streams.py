"""Calls on several HIP streams at once give the bits of the same calls made
one after another.

Every entry point takes the stream it runs on and keeps no state between
calls, so concurrent calls on different streams (forward, variants,
split-KV with its own workspace, backward) must not disturb each other.  The
kernels are deterministic, so each result is compared bit for bit with the
same call made alone on the default stream (whose results the parity tests
check against the oracle).
"""

import pytest
import torch

import io_aware_exact_fa1_amd as fa
import workloads
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def _dev(*ts):
    return [t.to("cuda") for t in ts]


def test_concurrent_streams_match_sequential_calls():
    require_gpu()
    qa, ka, va = _dev(*workloads.make_qkv(1, 8, 2000, 128, seed=71))
    qb, kb, vb = _dev(*workloads.make_qkv(1, 8, 1500, 64, seed=72))
    kb, vb = kb[:, :2].contiguous(), vb[:, :2].contiguous()  # Hkv = 2
    qc, _, _ = _dev(*workloads.make_qkv(1, 16, 3, 128, seed=73))
    _, kc, vc = _dev(*workloads.make_qkv(1, 2, 5000, 128, seed=74))
    g = torch.Generator(device="cpu")
    g.manual_seed(75)
    do = torch.randn(qa.shape, generator=g).to(torch.bfloat16).to("cuda")

    def calls():
        oa, la = fa.forward(qa, ka, va, causal=True)
        ob, lb = fa.forward_ex(qb, kb, vb, causal=True, window=300)
        oc, lc = fa.forward_split(qc, kc, vc, causal=True, nsplit=16)
        return oa, la, ob, lb, oc, lc

    say("streams: sequential reference on the default stream")
    oa, la, ob, lb, oc, lc = calls()
    grads = fa.backward(qa, ka, va, oa, la, do, causal=True)[:3]
    torch.cuda.synchronize()
    ref = [t.clone() for t in (oa, la, ob, lb, oc, lc, *grads)]

    streams = [torch.cuda.Stream() for _ in range(4)]
    for rep in range(3):
        say(f"streams: concurrent round {rep}")
        torch.cuda.synchronize()
        with torch.cuda.stream(streams[0]):
            ra = fa.forward(qa, ka, va, causal=True)
        with torch.cuda.stream(streams[1]):
            rb = fa.forward_ex(qb, kb, vb, causal=True, window=300)
        with torch.cuda.stream(streams[2]):
            rc = fa.forward_split(qc, kc, vc, causal=True, nsplit=16)
        with torch.cuda.stream(streams[3]):
            rg = fa.backward(qa, ka, va, ref[0], ref[1], do, causal=True)[:3]
        torch.cuda.synchronize()
        got = [*ra, *rb, *rc, *rg]
        names = ["O", "LSE", "O_ex", "LSE_ex", "O_split", "LSE_split", "dQ", "dK", "dV"]
        for name, x, y in zip(names, got, ref):
            assert torch.equal(x, y), (rep, name)
