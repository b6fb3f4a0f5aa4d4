"""Inputs past 2^31 elements (2^32 bytes in bf16) on every entry point.

The host checks accept up to 2^40 rows, so every offset into Q, K, V, O,
LSE and the workspaces must be formed in 64 bits.  Each case places its
heads so that one of them straddles element 2^31 of the largest tensor and
checks that head, its neighbours and the last head against the fp64 oracle
(same tolerances as the other parity tests).  The sequences are short
(72 rows: one ragged query tile, several key tiles at d = 64) so that the
many heads cost little time; the decode case instead has one long key
sequence per KV head.  Inputs are drawn on the device
(``workloads.make_qkv_device``); the checked heads are copied to the host.
"""

import math

import numpy as np
import pytest
import torch

import io_aware_exact_fa1_amd as fa
import workloads
from gpu_util import assert_close, f64, require_gpu, say
from oracle import attention_bwd_ref, attention_rows_ref
from oracle.variants import attention_ex_rows_ref

pytestmark = pytest.mark.gpu

E31 = 2 ** 31
N = 72  # one ragged 256-row query tile; key tiles of 64 (d = 128) or 128 (d = 64)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need(nbytes):
    """Skip (not fail) where the device cannot hold the case's tensors."""
    free, _ = torch.cuda.mem_get_info()
    if free < 1.1 * nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.1f} GiB of device memory, {free / 2**30:.1f} GiB free")


def _heads_to_check(n_heads, per_head):
    """The head that straddles element 2^31, its neighbours, the first and
    the last head."""
    h = E31 // per_head
    assert h * per_head < E31 < (h + 1) * per_head and h + 1 < n_heads
    return sorted({0, h - 1, h, h + 1, n_heads - 1})


@pytest.mark.parametrize("d,causal,dtype", [(128, False, torch.bfloat16), (128, True, torch.bfloat16),
                                            (64, True, torch.bfloat16), (64, False, torch.float32)])
def test_forward_past_2_31_elements(d, causal, dtype):
    H = E31 // (N * d) + 600
    B = 1
    assert B * H * N * d > E31
    _need(4 * B * H * N * d * (2 if dtype == torch.bfloat16 else 4))
    say("fa_fwd", tuple((B, H, N, d)), dtype, "causal" if causal else "non-causal")
    q, k, v = workloads.make_qkv_device(B, H, H, N, N, d, dtype, seed=31 + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(N)
    for h in _heads_to_check(B * H, N * d):
        o_ref, lse_ref = attention_rows_ref(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), scale, causal, rows)
        assert_close(f64(o[0, h]), f64(lse[0, h]), o_ref, lse_ref, dtype, f"fa_fwd d={d} head {h}")


def test_forward_ex_grouped_heads_past_2_31_elements():
    """GQA with the query tensors past 2^31 elements (K and V half that)."""
    d, Hkv, group = 128, E31 // (N * 128) // 2 + 300, 2
    Hq = Hkv * group
    _need((2 * Hq + 2 * Hkv) * N * d * 2)
    say("fa_fwd_ex", (1, Hq, Hkv, N, N, d), "causal")
    q, k, v = workloads.make_qkv_device(1, Hq, Hkv, N, N, d, seed=37)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward_ex(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(N)
    for h in _heads_to_check(Hq, N * d):
        o_ref, lse_ref = attention_ex_rows_ref(f64(q[0, h]), f64(k[0, h // group]), f64(v[0, h // group]), scale,
                                               True, 0, 0, rows)
        assert_close(f64(o[0, h]), f64(lse[0, h]), o_ref, lse_ref, torch.bfloat16, f"fa_fwd_ex head {h}")


def test_split_decode_past_2_31_key_elements():
    """One query per head against S keys per KV head, K and V past 2^31
    elements: the last KV head straddles the boundary."""
    d, Hkv, Hq = 128, 8, 64
    S = E31 // (Hkv * d) + 3001
    _need(2 * Hkv * S * d * 2)
    say("fa_fwd_split", (1, Hq, Hkv, 1, S, d), "causal nsplit=64")
    q, k, v = workloads.make_qkv_device(1, Hq, Hkv, 1, S, d, seed=41)
    assert k.numel() > E31 and (Hkv - 1) * S * d < E31
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward_split(q, k, v, causal=True, scale=scale, nsplit=64)
    torch.cuda.synchronize()
    group = Hq // Hkv
    for hk in (0, Hkv - 1):
        kh, vh = f64(k[0, hk]), f64(v[0, hk])
        for h in (hk * group, hk * group + group - 1):
            o_ref, lse_ref = attention_ex_rows_ref(f64(q[0, h]), kh, vh, scale, True, S - 1, 0, [0])
            assert_close(f64(o[0, h]), f64(lse[0, h]), o_ref, lse_ref, torch.bfloat16, f"fa_fwd_split head {h}")


def test_backward_past_2_31_elements():
    from test_bwd_parity import BWD_MAX, BWD_MEAN

    d = 128
    H = E31 // (N * d) + 600
    _need(8 * H * N * d * 2)
    say("fa_bwd", (1, H, N, d), "causal")
    q, k, v = workloads.make_qkv_device(1, H, H, N, N, d, seed=43)
    g = torch.Generator(device="cuda")
    g.manual_seed(47)
    do = torch.randn(q.shape, generator=g, dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    dq, dk, dv, _ = fa.backward(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    for h in _heads_to_check(H, N * d):
        refs = attention_bwd_ref(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(do[0, h]), scale, True)
        for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
            err = np.abs(f64(got[0, h]) - ref)
            s = max(1.0, float(np.abs(ref).max()))
            say(f"fa_bwd head {h} {name}: max {err.max():.3e} mean {err.mean():.3e} (scale {s:.2f})")
            assert np.all(np.isfinite(f64(got[0, h])))
            assert err.max() <= BWD_MAX * s and err.mean() <= BWD_MEAN * s, (h, name)
