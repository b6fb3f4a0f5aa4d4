"""The forward entry points captured in a HIP graph (torch.cuda.CUDAGraph):
they allocate nothing, issue no memset and launch only their own kernels
on the given stream, so a captured call replays correctly.  Each replay
runs on new inputs written into the captured buffers, with eager work of
the program in between, and must equal the eager call on the same inputs
bit for bit."""

import pytest
import torch

from gpu_util import require_gpu, say
import io_aware_exact_fa1_amd as fa

pytestmark = pytest.mark.gpu


def _fill(bufs, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    for b in bufs:
        b.copy_(torch.randn(b.shape, generator=g, dtype=torch.float32).to(b.dtype))


def _replays(call, inputs, outputs, what, n=3):
    """Capture call() once, then for n fresh inputs compare the replay with
    the eager call."""
    _fill(inputs, 0)
    call()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(n):
        say(f"{what} replay {r}")
        _fill(inputs, 100 + r)
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in outputs]
        # eager work between replays: scramble the outputs, then the eager call
        for x in outputs:
            x.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        for a, b in zip(got, outputs):
            assert torch.equal(a, b), f"{what}: replay {r} differs from the eager call"


@pytest.mark.parametrize("d,causal", [(128, True), (64, False)])
def test_fa_fwd_in_a_graph(d, causal):
    require_gpu()
    B, H, N = 1, 4, 777
    q, k, v = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def call():
        st = fa.fa_fwd(q, k, v, o, lse, B, H, N, d, d ** -0.5, causal, torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK

    _replays(call, [q, k, v], [o, lse], f"fa_fwd d={d} causal={causal}")


@pytest.mark.parametrize("Hq,Hkv,T,S,window", [(16, 4, 300, 1000, 0), (8, 2, 64, 640, 100)])
def test_fa_fwd_ex_in_a_graph(Hq, Hkv, T, S, window):
    require_gpu()
    B, d = 2, 128
    q = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device="cuda")
    k, v = (torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")

    def call():
        st = fa.fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, T, S, d, d ** -0.5, 1, S - T, window,
                          torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK

    _replays(call, [q, k, v], [o, lse], f"fa_fwd_ex Hq={Hq} Hkv={Hkv} T={T} S={S} window={window}")


@pytest.mark.parametrize("Hq,Hkv,T,S,nsplit,d", [
    (32, 4, 1, 5000, 16, 128),     # small-tile partial kernel + merge
    (8, 8, 4, 3000, 1, 64),        # small-tile kernel, one chunk (no merge)
    (4, 2, 300, 2000, 4, 128),     # large-tile split mode + merge
])
def test_fa_fwd_split_in_a_graph(Hq, Hkv, T, S, nsplit, d):
    require_gpu()
    B = 2
    q = torch.empty((B, Hq, T, d), dtype=torch.bfloat16, device="cuda")
    k, v = (torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    G = fa.fa_split_chunks(S, nsplit)
    ws_o = torch.empty((G, B, Hq, T, d), dtype=torch.float32, device="cuda")
    ws_l = torch.empty((G, B, Hq, T), dtype=torch.float32, device="cuda")

    def call():
        st = fa.fa_fwd_split(q, k, v, o, lse, B, Hq, Hkv, T, S, d, d ** -0.5, 1, S - T, 0, nsplit, ws_o, ws_l,
                             torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK

    _replays(call, [q, k, v], [o, lse], f"fa_fwd_split Hq={Hq} Hkv={Hkv} T={T} S={S} nsplit={nsplit} d={d}")
