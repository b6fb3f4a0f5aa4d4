"""GPU checks of the bf16 forward's exponent reference and of the paired
causal work units, against the fp64 oracle.

The kernel fixes a row's exponent reference at the max of its first key
tile and keeps every later weight at most 2^16 by taking the running-max
step of the recurrence ("15. FlashAttention", section "Online softmax:
normalize as you go") on the tiles where a row's scores rise further.  The
cases here give the rows large values of V together with a score rise of
about 30 or 40 in log2 units after the first tile.  With weights allowed to
reach 2^40 instead, the second case (2^40 times |V| = 2^85, summed over
hundreds of keys) would leave the fp32 range of the accumulator, while the
recurrence stays finite.

The paired cases use B*H*T_r > 256 query tiles (T_r = ceil(N / 256)), so
that each causal work unit runs a heavy query tile and then a light one
whose keys are walked from last to first.
"""

import math

import numpy as np
import pytest
import torch

import io_aware_exact_fa1_amd as fa
import workloads
from gpu_util import assert_close, f64, require_gpu, run_gpu, say
from oracle import attention_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("vexp,lift", [(70, 21.0), (85, 28.0)], ids=["v2^70_rise30", "v2^85_rise40"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_large_values_after_a_rise(d, causal, vexp, lift):
    """|V| about 2^vexp; every row of head 0 and some of head 1 see their
    scores rise by ``lift`` nats (about 30 or 40 in log2 units) from key 300
    on.  O scales exactly with V (a power of two), so O * 2^-vexp is checked
    against the oracle on the unscaled V with the bf16 tolerances."""
    N = 700
    rows = [(0, t) for t in range(N)] + [(1, t) for t in range(0, N, 7)]
    q, k, v = workloads.make_jump_qkv(1, 2, 2, N, N, d, rows, key0=300, lift=lift, seed=71 + d)
    vs = (v.float() * 2.0 ** vexp).to(torch.bfloat16)
    assert np.array_equal(f64(vs) * 2.0 ** -vexp, f64(v))  # the scaling is exact
    scale = 1.0 / math.sqrt(d)
    say("large values after a rise", d, causal, vexp, lift)
    o, lse = run_gpu(q, k, vs, causal, scale)
    o_ref, lse_ref = attention_ref(f64(q), f64(k), f64(v), scale, causal)
    assert_close(f64(o) * 2.0 ** -vexp, f64(lse), o_ref, lse_ref, torch.bfloat16,
                 f"|V|~2^{vexp} lift={lift} d={d} causal={causal}")
    assert lse_ref[0, 0, N - 1] > lift - 5.0  # the rows did rise


def _paired_shape():
    # 96 heads x 5 query tiles = 480 > 256: causal units pair tiles (4, 0),
    # (3, 1) and leave tile 2 alone; the light tiles 0 and 1 walk their keys
    # from last to first
    return 1, 96, 1100


@pytest.mark.parametrize("d", [64, 128])
def test_paired_causal_future_keys_contribute_exactly_zero(d):
    """On the paired causal path, rows < r are bit-identical when K and V
    rows >= r are replaced by other finite values (including +-1e4)."""
    B, H, N = _paired_shape()
    q, k, v = (x.cuda() for x in workloads.make_qkv(B, H, N, d, torch.bfloat16, seed=61 + d))
    o0, l0 = fa.forward(q, k, v, causal=True)
    for r in (1, 100, 255, 256, 300, 511, 600, 1023, 1099):
        say("paired future keys", d, r)
        k2, v2 = k.clone(), v.clone()
        g = torch.Generator(device="cpu").manual_seed(r)
        k2[:, :, r:] = (torch.randn(k2[:, :, r:].shape, generator=g) * 1e4).to(torch.bfloat16).cuda()
        v2[:, :, r:] = (-torch.randn(v2[:, :, r:].shape, generator=g) * 1e4).to(torch.bfloat16).cuda()
        o1, l1 = fa.forward(q, k2, v2, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, :, :r], o0[:, :, :r]), r
        assert torch.equal(l1[:, :, :r], l0[:, :, :r]), r


# rows of the light tiles 0 (rows 0..255) and 1 (256..511) of paired units,
# at several lanes and waves, plus rows of the heavy tiles and of tile 2
PAIRED_JUMP_ROWS = [(0, 5), (0, 63), (0, 200), (1, 256), (1, 300), (1, 511), (7, 400), (95, 255),
                    (3, 700), (3, 1099), (50, 600)]


@pytest.mark.parametrize("key0,key1", [(150, None), (0, 100)], ids=["rise_late", "rise_early"])
@pytest.mark.parametrize("d", [64, 128])
def test_jump_rows_in_paired_units(d, key0, key1):
    """The listed rows see their scores rise by 60 nats on keys key0 ..
    key1.  With keys 0 .. 99 lifted, a light tile meets the lifted keys at
    the end of its descending walk, after its reference was set on lower
    scores; with keys from 150 on lifted, the heavy tiles meet them after
    their first tile.  Every row of every head against the oracle."""
    B, H, N = _paired_shape()
    q, k, v = workloads.make_jump_qkv(B, H, H, N, N, d, PAIRED_JUMP_ROWS, key0=key0, key1=key1, seed=81 + d)
    scale = 1.0 / math.sqrt(d)
    say("paired jump rows", d, key0, key1)
    o, lse = run_gpu(q, k, v, True, scale)
    o_ref, lse_ref = attention_ref(f64(q), f64(k), f64(v), scale, True)
    assert_close(f64(o), f64(lse), o_ref, lse_ref, torch.bfloat16, f"paired jump d={d} keys {key0}..{key1}")
    for h, t in PAIRED_JUMP_ROWS:
        if t >= key0:
            assert lse_ref[0, h, t] > 50.0, (h, t)
    # the other rows saw no rise
    assert float(np.median(lse_ref)) < 15.0
