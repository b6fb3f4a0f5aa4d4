"""fa_fwd_ex (grouped K/V heads, query offset, sliding window) on the GPU,
through the C ABI, against the fp64 variants oracle.  Tolerances are the
forward's bf16 bounds (max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <=
1e-3)."""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, f64, require_gpu, say
from oracle.variants import attention_ex_ref, attention_ex_rows_ref
import io_aware_exact_fa1_amd as fa
import workloads

pytestmark = pytest.mark.gpu


def _qkv(B, Hq, Hkv, T, S, d, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, Hq, T, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def _run(q, k, v, causal, offset=None, window=0, scale=None):
    o, lse = fa.forward_ex(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, offset=offset,
                           window=window)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


def _check(q, k, v, causal, offset, window, what):
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d)
    say(what)
    o, lse = _run(q, k, v, causal, offset, window)
    ro, rl = attention_ex_ref(f64(q), f64(k), f64(v), scale, causal, offset, window)
    assert_close(o, lse, ro, rl, torch.bfloat16, what)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_plain_case_equals_fa_fwd_bitwise(d, causal):
    """Hq = Hkv, T = S, offset 0, no window: the same bits as fa_fwd."""
    require_gpu()
    q, k, v = _qkv(2, 3, 3, 700, 700, d, seed=11)
    say(f"plain d={d} causal={causal}")
    o1, l1 = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    o2, l2 = fa.forward_ex(q.cuda(), k.cuda(), v.cuda(), causal=causal, offset=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_gqa(group, causal):
    require_gpu()
    hkv = 2
    q, k, v = _qkv(2, hkv * group, hkv, 333, 333, 128, seed=20 + group)
    _check(q, k, v, causal, 0 if causal else None, 0, f"gqa group={group} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,S", [(1, 300), (37, 300), (256, 1000), (300, 301), (1000, 1000)])
def test_chunked_prefill_and_decode(T, S, d):
    """Causal, queries at the newest positions (offset S - T)."""
    require_gpu()
    q, k, v = _qkv(1, 4, 2, T, S, d, seed=T + S)
    _check(q, k, v, True, None, 0, f"prefill T={T} S={S} d={d}")


def test_explicit_offsets():
    require_gpu()
    q, k, v = _qkv(1, 2, 1, 100, 700, 128, seed=5)
    for off in (0, 1, 63, 64, 300, 600):
        _check(q, k, v, True, off, 0, f"offset={off}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [1, 31, 64, 100, 257, 5000])
def test_sliding_window(window, d):
    require_gpu()
    q, k, v = _qkv(1, 4, 4, 600, 600, d, seed=window + d)
    _check(q, k, v, True, 0, window, f"window={window} d={d}")


def test_window_with_offset_and_gqa():
    require_gpu()
    q, k, v = _qkv(2, 8, 2, 200, 900, 128, seed=99)
    for off, w in ((700, 128), (350, 33), (0, 1000)):
        _check(q, k, v, True, off, w, f"offset={off} window={w}")


@pytest.mark.parametrize("T,S", [(100, 700), (700, 100), (1, 4096)])
def test_cross_attention(T, S):
    """No causal mask: every query sees all S keys, whatever T is."""
    require_gpu()
    q, k, v = _qkv(1, 2, 1, T, S, 64, seed=T * 7 + S)
    _check(q, k, v, False, None, 0, f"cross T={T} S={S}")


def test_window_keys_outside_do_not_matter():
    """Keys before the window of every row may hold anything, bitwise."""
    require_gpu()
    N, W = 512, 64
    q, k, v = _qkv(1, 2, 2, N, N, 128, seed=3)
    o1, l1 = _run(q, k, v, True, 0, W)
    k2, v2 = k.clone(), v.clone()
    r0 = 300  # rows >= r0 never see keys < r0 - W + 1
    k2[:, :, :r0 - W + 1] = (torch.randn_like(k2[:, :, :r0 - W + 1].float()) * 30).to(torch.bfloat16)
    v2[:, :, :r0 - W + 1] = -v2[:, :, :r0 - W + 1]
    o2, l2 = _run(q, k2, v2, True, 0, W)
    assert np.array_equal(o1[:, :, r0:], o2[:, :, r0:]) and np.array_equal(l1[:, :, r0:], l2[:, :, r0:])


def test_long_context_gqa_window_sampled():
    """Hq = 64 over Hkv = 8, N = 16384, d = 128, causal, window 4096: sampled rows."""
    require_gpu()
    B, Hq, Hkv, N, d, W = 1, 64, 8, 16384, 128, 4096
    q, k, v = _qkv(B, Hq, Hkv, N, N, d, seed=123)
    say("long context gqa window")
    o, lse = _run(q, k, v, True, 0, W)
    rows = np.array([0, 1, 4095, 4096, 8191, 12345, 16383])
    for h in (0, 37, 63):
        ro, rl = attention_ex_rows_ref(f64(q[0, h]), f64(k[0, h // 8]), f64(v[0, h // 8]), 1 / np.sqrt(d), True,
                                       0, W, rows)
        assert_close(o[0, h, rows], lse[0, h, rows], ro, rl, torch.bfloat16, f"h={h}")


@pytest.mark.parametrize("d", [64, 128])
def test_climbing_scores_take_the_exact_pass(d):
    """Keys ramped along the mean query direction of each K/V group's first
    head, so that the scores of many rows (of every head, scattered over
    lanes and waves) climb by up to hundreds of nats: the rows that outgrow
    the fixed reference of their first tile are redone by the exact pass,
    with grouped heads, an offset and a window."""
    require_gpu()
    B, Hq, Hkv, T, S = 1, 4, 2, 300, 1500
    g = torch.Generator(device="cpu")
    g.manual_seed(77 + d)
    q = torch.randn((B, Hq, T, d), generator=g)
    k = torch.randn((B, Hkv, S, d), generator=g)
    v = torch.randn((B, Hkv, S, d), generator=g)
    qs = q[:, ::Hq // Hkv, :]                               # every row of the group's first head
    u = qs.mean(dim=2, keepdim=True)
    u = u / u.norm(dim=-1, keepdim=True)
    per = 300.0 / (qs.norm(dim=-1).mean() / np.sqrt(d))
    k = k + per * torch.linspace(0, 1, S)[None, None, :, None] * u
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    for off, w in ((S - T, 0), (700, 500), (S - T, 64)):
        _check(q, k, v, True, off, w, f"climbing d={d} offset={off} window={w}")


# (head, row) pairs whose scores jump at key 800: rows at lanes 4, 3, 1, 11,
# 8 and 3 of their wave, one of them alone in head 3
EX_JUMP_ROWS = [(0, 100), (0, 131), (1, 257), (1, 299), (2, 200), (3, 163)]


@pytest.mark.parametrize("d", [64, 128])
def test_score_jump_some_rows(d):
    """Only the rows in EX_JUMP_ROWS see their scores rise by 60 nats at key
    800 (past the reference of the first tile each of them sees), with
    grouped heads, an offset and a window: those rows alone take the
    running-max step."""
    require_gpu()
    B, Hq, Hkv, T, S = 1, 4, 2, 300, 1500
    q, k, v = workloads.make_jump_qkv(B, Hq, Hkv, T, S, d, EX_JUMP_ROWS, key0=800, seed=41 + d)
    for off, w in ((S - T, 0), (700, 500)):
        _check(q, k, v, True, off, w, f"jump rows d={d} offset={off} window={w}")


@pytest.mark.parametrize("d", [64, 128])
def test_long_cross_attention_rounds(d):
    """T = 8500 queries over S = 3000 keys without a mask (34 query tiles per
    head, more than one XCD runs at once), grouped heads; sampled rows
    against the oracle."""
    require_gpu()
    q, k, v = _qkv(1, 4, 2, 8500, 3000, d, seed=950 + d)
    say(f"long cross-attention d={d}")
    o, lse = fa.forward_ex(q.cuda(), k.cuda(), v.cuda(), causal=False)
    torch.cuda.synchronize()
    rows = np.union1d(workloads.sample_rows(8500, 64, seed=d), np.array([8191, 8192, 8499]))
    for h in (0, 3):
        ro, rl = attention_ex_rows_ref(f64(q[0, h]), f64(k[0, h // 2]), f64(v[0, h // 2]), 1 / np.sqrt(d), False,
                                       0, 0, rows)
        assert_close(f64(o[0, h])[rows], f64(lse[0, h])[rows], ro, rl, torch.bfloat16, f"cross d={d} h={h}")
