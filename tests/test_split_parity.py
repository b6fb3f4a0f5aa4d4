"""fa_fwd_split (split-KV, flash-decoding) on the GPU, through the C ABI,
against the fp64 variants oracle: the per-chunk partials (O_g, L_g) the
first kernel leaves in the workspace, and the merged result.  Tolerances are
the forward's bf16 bounds (max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE|
<= 1e-3); which partials are empty (L_g = -inf, O_g = 0) is a masking
decision and must match exactly."""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, f64, require_gpu, say
from oracle.variants import attention_ex_ref, attention_ex_rows_ref, attention_split_ref, merge_partials_ref
import io_aware_exact_fa1_amd as fa
import workloads

pytestmark = pytest.mark.gpu


def _qkv(B, Hq, Hkv, T, S, d, seed, ramp=0.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, Hq, T, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, S, d), generator=g, dtype=torch.float32)
    if ramp:
        # for row 0 of the first head of each K/V group, scores that climb
        # by about `ramp` nats from the first key to the last: later keys
        # outgrow any reference taken from the first tiles
        qs = q[:, ::Hq // Hkv, :1]                           # [B, Hkv, 1, d]
        u = qs / qs.norm(dim=-1, keepdim=True)
        per = ramp / (qs.norm(dim=-1, keepdim=True) / np.sqrt(d))
        k = k + per * torch.linspace(0, 1, S)[None, None, :, None] * u
    return (x.to(torch.bfloat16) for x in (q, k, v))


def _chunk(S, nsplit):
    return -(-(-(-S // nsplit)) // 128) * 128


def _run(q, k, v, causal, offset, window, nsplit):
    B, Hq, T, d = q.shape
    S = k.shape[2]
    G = fa.fa_split_chunks(S, nsplit)
    ws_o = torch.full((G, B, Hq, T, d), float("nan"), dtype=torch.float32, device="cuda")
    ws_l = torch.full((G, B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    o, lse = fa.forward_split(q.cuda(), k.cuda(), v.cuda(), causal=causal, offset=offset, window=window,
                              nsplit=nsplit, workspace=(ws_o, ws_l))
    torch.cuda.synchronize()
    return f64(o), f64(lse), f64(ws_o), f64(ws_l)


def _check(q, k, v, causal, offset, window, nsplit, what, partials=True):
    d = q.shape[-1]
    S, T = k.shape[2], q.shape[2]
    scale = 1.0 / np.sqrt(d)
    G = fa.fa_split_chunks(S, nsplit)
    say(f"{what} G={G}")
    o, lse, wo, wl = _run(q, k, v, causal, offset, window, nsplit)
    ro, rl = attention_ex_ref(f64(q), f64(k), f64(v), scale, causal, offset, window)
    assert_close(o, lse, ro, rl, torch.bfloat16, what)
    if partials and G > 1:
        po, pl = attention_split_ref(f64(q), f64(k), f64(v), scale, causal, offset, window, _chunk(S, nsplit))
        assert po.shape[0] == G
        empty = np.isneginf(pl)
        assert np.array_equal(np.isneginf(wl), empty), f"{what}: empty partials differ"
        assert np.all(wo[empty] == 0.0), f"{what}: empty partial O_g not zero"
        full = ~empty
        assert_close(wo[full], wl[full], po[full], pl[full], torch.bfloat16, what + " partials")
        # the merge kernel: the oracle's merge of the kernel's own partials,
        # up to the final bf16 rounding of O (half an ulp: at most 2^-8
        # relative, bf16 keeping 8 significant bits)
        # and fp32 rounding of the weights and of LSE
        mo, ml = merge_partials_ref(wo, wl)
        assert np.all(np.abs(mo - o) <= 2.0 ** -8 * np.abs(mo) + 1e-5), what + " merge O"
        assert np.all(np.abs(ml - lse) <= 1e-5 + 1e-6 * np.abs(ml)), what + " merge LSE"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", [1, 129, 300, 1000, 4096])
@pytest.mark.parametrize("nsplit", [2, 3, 8])
def test_decode(S, nsplit, d):
    """T = 1 at the newest position (offset S - 1), grouped K/V heads."""
    require_gpu()
    q, k, v = _qkv(2, 8, 2, 1, S, d, seed=S * 13 + nsplit + d)
    _check(q, k, v, True, None, 0, nsplit, f"decode S={S} nsplit={nsplit} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,S", [(37, 300), (256, 1000), (300, 301), (700, 700)])
def test_chunked_prefill(T, S, d):
    """Causal queries at the newest positions: rows of one tile see
    different numbers of keys of the last chunks, some none."""
    require_gpu()
    q, k, v = _qkv(1, 4, 2, T, S, d, seed=T + S + d)
    for nsplit in (2, 5):
        _check(q, k, v, True, None, 0, nsplit, f"prefill T={T} S={S} d={d} nsplit={nsplit}")


@pytest.mark.parametrize("d", [64, 128])
def test_window_and_offsets(d):
    require_gpu()
    q, k, v = _qkv(1, 4, 1, 100, 900, d, seed=7 + d)
    for off, w, ns in ((800, 0, 4), (800, 128, 4), (350, 33, 3), (0, 1000, 7), (500, 300, 7)):
        _check(q, k, v, True, off, w, ns, f"offset={off} window={w} nsplit={ns} d={d}")


@pytest.mark.parametrize("T,S", [(1, 4096), (100, 700), (700, 100)])
def test_cross_attention(T, S):
    """No causal mask: every chunk is seen by every row (no empty partial)."""
    require_gpu()
    q, k, v = _qkv(1, 2, 1, T, S, 128, seed=T * 3 + S)
    _check(q, k, v, False, None, 0, 4, f"cross T={T} S={S}")


def test_single_chunk_is_fa_fwd_ex_bitwise():
    """G = 1 (nsplit 1) with more than 32 query rows per K/V head: the call
    is fa_fwd_ex itself, workspace unused."""
    require_gpu()
    q, k, v = _qkv(1, 4, 2, 17, 700, 128, seed=1)
    say("single chunk")
    o1, l1 = fa.forward_ex(q.cuda(), k.cuda(), v.cuda(), causal=True)
    o2, l2 = fa.forward_split(q.cuda(), k.cuda(), v.cuda(), causal=True, nsplit=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_climbing_scores_take_the_exact_path():
    """Scores that climb by hundreds of nats along the keys: rows whose
    later keys outgrow the first tile's reference take the running-max step
    inside each chunk, partials included."""
    require_gpu()
    for d, T, S in ((128, 1, 4096), (64, 1, 4096), (128, 64, 2000)):
        q, k, v = _qkv(1, 4, 2, T, S, d, seed=d + T, ramp=300.0)
        _check(q, k, v, True, None, 0, 4, f"climbing d={d} T={T} S={S}")


@pytest.mark.parametrize("d", [64, 128])
def test_score_jump_some_rows(d):
    """Only a few scattered rows see their scores rise by 60 nats at key 800,
    inside the second of three chunks: those rows raise their reference in
    that chunk's partial (large-tile split path, then the merge)."""
    require_gpu()
    rows = [(0, 100), (0, 131), (1, 257), (1, 299), (2, 200), (3, 163)]
    q, k, v = workloads.make_jump_qkv(1, 4, 2, 300, 1500, d, rows, key0=800, seed=51 + d)
    for off, w in ((1200, 0), (700, 500)):
        _check(q, k, v, True, off, w, 3, f"jump rows d={d} offset={off} window={w}")


def test_deterministic_and_workspace_reuse():
    """Two calls give the same bits; a smaller call in the same (larger)
    workspace is still right."""
    require_gpu()
    q, k, v = _qkv(2, 8, 2, 3, 3000, 128, seed=5)
    say("determinism")
    a = _run(q, k, v, True, None, 0, 6)
    b = _run(q, k, v, True, None, 0, 6)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    G = fa.fa_split_chunks(3000, 6)
    ws = (torch.empty((G, 2, 8, 3, 128), dtype=torch.float32, device="cuda"),
          torch.empty((G, 2, 8, 3), dtype=torch.float32, device="cuda"))
    fa.forward_split(q.cuda(), k.cuda(), v.cuda(), causal=True, nsplit=6, workspace=ws)
    q2, k2, v2 = _qkv(1, 2, 1, 1, 1000, 128, seed=6)
    o, lse = fa.forward_split(q2.cuda(), k2.cuda(), v2.cuda(), causal=True, nsplit=3, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = attention_ex_ref(f64(q2), f64(k2), f64(v2), 1 / np.sqrt(128), True)
    assert_close(f64(o), f64(lse), ro, rl, torch.bfloat16, "reuse")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv,T", [(1, 1, 32), (4, 1, 8), (8, 1, 3), (2, 2, 5), (16, 2, 2), (32, 4, 1)])
def test_small_tile_rows(Hq, Hkv, T, d):
    """Up to 32 query rows per K/V head (group * T <= 32): the small-tile
    kernel, whose 32 columns hold the group's heads times the T rows;
    causal with the newest positions, with an offset and a window, and
    non-causal; one chunk (O and LSE written directly) and several."""
    require_gpu()
    S = 1000
    q, k, v = _qkv(2, Hq, Hkv, T, S, d, seed=Hq * 100 + T + d)
    for causal, off, w, ns in ((True, None, 0, 1), (True, None, 0, 4), (True, 500, 0, 3), (True, 700, 77, 5),
                               (True, None, 300, 8), (False, None, 0, 1), (False, None, 0, 6)):
        _check(q, k, v, causal, off, w, ns, f"small Hq={Hq} Hkv={Hkv} T={T} d={d} causal={causal} "
               f"offset={off} window={w} nsplit={ns}")


@pytest.mark.parametrize("S", [1, 31, 32, 33, 95, 128, 129, 4097])
def test_small_tile_tails(S):
    """Ragged key counts around the 32-key tiles and 128-key chunks."""
    require_gpu()
    q, k, v = _qkv(1, 8, 2, min(2, S), S, 128, seed=S)
    for ns in (1, 2, 7):
        _check(q, k, v, True, None, 0, ns, f"tails S={S} nsplit={ns}")


@pytest.mark.parametrize("nsplit", [8, 16, 64])
def test_long_context_decode(nsplit):
    """Decode against a 16384-key cache: Hq = 64 over Hkv = 8, d = 128,
    every head, with the partials."""
    require_gpu()
    q, k, v = _qkv(1, 64, 8, 1, 16384, 128, seed=123 + nsplit)
    _check(q, k, v, True, None, 0, nsplit, f"long decode nsplit={nsplit}")


def test_long_context_chunked_prefill_window():
    """256 new queries after 16128 cached keys, window 4096, Hq = 64 over
    Hkv = 8."""
    require_gpu()
    q, k, v = _qkv(1, 64, 8, 256, 16384, 128, seed=77)
    _check(q, k, v, True, None, 4096, 8, "long prefill window", partials=False)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_many_groups(d):
    """B = 8 sequences, 64 query heads over 4 K/V heads (groups of 16, so
    32 columns at T = 2), S = 3000, several chunks: 8 * 4 * G workgroups of
    the small-tile kernel; every 9th head against the oracle."""
    require_gpu()
    B, Hq, Hkv, T, S = 8, 64, 4, 2, 3000
    q, k, v = _qkv(B, Hq, Hkv, T, S, d, seed=5150 + d)
    say(f"decode many groups d={d}")
    o, lse, _, _ = _run(q, k, v, True, None, 0, 6)
    scale = 1.0 / np.sqrt(d)
    for idx in range(0, B * Hq, 9):
        b, h = divmod(idx, Hq)
        ro, rl = attention_ex_rows_ref(f64(q[b, h]), f64(k[b, h // (Hq // Hkv)]), f64(v[b, h // (Hq // Hkv)]), scale,
                                       True, S - T, 0, np.arange(T))
        assert_close(o[b, h], lse[b, h], ro, rl, torch.bfloat16, f"b={b} h={h}")
