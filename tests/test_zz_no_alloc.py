"""fa_fwd_split_noalloc (partials in the library's static device scratch)
against fa_fwd_split (partials in caller workspaces): the same kernels, so
the results must agree bit for bit.  Calls follow one another with
decreasing sizes, so that a later call runs on a scratch still holding a
larger call's partials; every partial the merge reads must have been
written by the same call."""

import math

import pytest
import torch

import io_aware_exact_fa1_amd as fa
from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, T, S, d, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, Hq, T, d), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((B, Hkv, S, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, Hkv, S, d), generator=g).to(torch.bfloat16).cuda()
    return q, k, v


def _both(B, Hq, Hkv, T, S, d, causal, window, nsplit, seed):
    q, k, v = _inputs(B, Hq, Hkv, T, S, d, seed)
    scale = 1.0 / math.sqrt(d)
    offset = S - T
    G = fa.fa_split_chunks(S, nsplit)
    ws_o = torch.empty((G, B, Hq, T, d), dtype=torch.float32, device="cuda")
    ws_l = torch.empty((G, B, Hq, T), dtype=torch.float32, device="cuda")
    o1 = torch.empty_like(q)
    l1 = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    say("noalloc", B, Hq, Hkv, T, S, d, causal, window, nsplit, "G", G)
    st = fa.fa_fwd_split(q, k, v, o1, l1, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit, ws_o, ws_l)
    assert st == fa.FA_OK, fa.fa_strerror(st)
    st = fa.fa_fwd_split_noalloc(q, k, v, o2, l2, B, Hq, Hkv, T, S, d, scale, causal, offset, window, nsplit)
    assert st == fa.FA_OK, fa.fa_strerror(st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "O differs"
    assert torch.equal(l1, l2), "LSE differs"
    assert bool(torch.isfinite(o2).all()) and bool(torch.isfinite(l2).all())


# (B, Hq, Hkv, T, S, d, causal, window, nsplit): each a smaller call than the
# one before on its path; decode (small-tile partial kernel) and chunked
# prefill (large-tile partial kernel), ragged key counts
DECODE = [(4, 64, 8, 1, 16384, 128, True, 0, 32), (1, 16, 4, 2, 3001, 128, True, 0, 8),
          (1, 8, 8, 1, 900, 64, False, 0, 4)]
PREFILL = [(1, 8, 2, 300, 5000, 128, True, 0, 4), (1, 4, 1, 100, 2100, 64, True, 700, 3)]


def test_noalloc_matches_split_decode():
    require_gpu()
    for i, case in enumerate(DECODE):
        _both(*case, seed=700 + i)


def test_noalloc_matches_split_prefill():
    require_gpu()
    for i, case in enumerate(PREFILL):
        _both(*case, seed=800 + i)


def test_noalloc_single_chunk_and_limit():
    """One chunk needs no scratch (the direct kernels); a call whose partials
    exceed the scratch is refused before any launch, leaving O untouched."""
    require_gpu()
    _both(1, 8, 2, 1, 100, 128, True, 0, 8, seed=900)
    B, Hq, Hkv, T, S, d = 1, 64, 64, 2048, 2048, 128   # 4 chunks: 4 * 131072 * 129 * 4 bytes = 270 MB
    q, k, v = _inputs(B, Hq, Hkv, T, S, d, 901)
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, T), 7.0, device="cuda")
    st = fa.fa_fwd_split_noalloc(q, k, v, o, lse, B, Hq, Hkv, T, S, d, 0.1, 1, 0, 0, 4)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_SCRATCH
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
