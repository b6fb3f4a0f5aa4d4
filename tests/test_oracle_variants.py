"""The variants oracle (GQA, query offset, sliding window) against pins that
come from outside it, and the pins against planted mistakes."""

import math

import numpy as np
import pytest

from oracle import attention_ref
from oracle.variants import attention_ex_ref, attention_ex_rows_ref


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b))))
    assert err <= tol, f"{what}: {err:.3e} > {tol:.1e}"


def _loop_attention(q, k, v, scale, visible):
    """One head with scalar loops and math.fsum: row i over keys j with visible(i, j)."""
    T, S = q.shape[0], k.shape[0]
    o = np.zeros((T, v.shape[1]))
    lse = np.zeros(T)
    for i in range(T):
        keys = [j for j in range(S) if visible(i, j)]
        s = [scale * math.fsum(q[i, e] * k[j, e] for e in range(q.shape[1])) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(wj * v[j, c] for wj, j in zip(w, keys)) / tot
        lse[i] = mx + math.log(tot)
    return o, lse


# ---------------------------------------------------------------- pins
def pin_square_reduces_to_plain(ex):
    """T = S, offset 0, no window, one KV head per query head: the plain
    (already pinned) definition."""
    r = _rng(1)
    q, k, v = (r.standard_normal((2, 3, 37, 8)) for _ in range(3))
    for causal in (False, True):
        o, lse = ex(q, k, v, 0.4, causal, 0, 0)
        o2, lse2 = attention_ref(q, k, v, 0.4, causal)
        _close(o, o2, 1e-13, "O"); _close(lse, lse2, 1e-13, "LSE")


def pin_window_one(ex):
    """W = 1: each row sees only the key at its own position:
    O_i = v_{p_i}, LSE_i = scale q_i . k_{p_i}."""
    r = _rng(2)
    T, S, d = 9, 20, 5
    q = r.standard_normal((1, 1, T, d)); k = r.standard_normal((1, 1, S, d)); v = r.standard_normal((1, 1, S, d))
    off = S - T
    o, lse = ex(q, k, v, 0.7, True, off, 1)
    for i in range(T):
        p = off + i
        _close(o[0, 0, i], v[0, 0, p], 1e-14, "O")
        _close(lse[0, 0, i], 0.7 * q[0, 0, i] @ k[0, 0, p], 1e-13, "LSE")


def pin_window_brute_force(ex):
    """Windows against scalar loops over exactly the keys p-W+1 .. p."""
    r = _rng(3)
    T, S, d = 7, 12, 3
    q = r.standard_normal((1, 1, T, d)); k = r.standard_normal((1, 1, S, d)); v = r.standard_normal((1, 1, S, d))
    for off in (0, 2, S - T):
        for W in (2, 3, 5, 40):
            o, lse = ex(q, k, v, 0.9, True, off, W)
            o2, lse2 = _loop_attention(q[0, 0], k[0, 0], v[0, 0], 0.9,
                                       lambda i, j, off=off, W=W: off + i - W + 1 <= j <= off + i)
            _close(o[0, 0], o2, 1e-13, f"O off={off} W={W}"); _close(lse[0, 0], lse2, 1e-13, "LSE")


def pin_chunked_prefill(ex):
    """T < S with the default offset S - T: the last T rows of causal square
    attention over S positions whose last T queries are q."""
    r = _rng(4)
    S, T, d = 30, 8, 6
    qfull = r.standard_normal((1, 2, S, d)); k = r.standard_normal((1, 2, S, d)); v = r.standard_normal((1, 2, S, d))
    o, lse = ex(qfull[:, :, S - T:], k, v, 0.5, True, None, 0)
    o2, lse2 = attention_ref(qfull, k, v, 0.5, True)
    _close(o, o2[:, :, S - T:], 1e-13, "O"); _close(lse, lse2[:, :, S - T:], 1e-13, "LSE")


def pin_decode_row(ex):
    """T = 1 at the last position sees every key: a one-row non-causal
    softmax, against scalar loops."""
    r = _rng(5)
    S, d = 17, 4
    q = r.standard_normal((1, 1, 1, d)); k = r.standard_normal((1, 1, S, d)); v = r.standard_normal((1, 1, S, d))
    o, lse = ex(q, k, v, 1.1, True, None, 0)
    o2, lse2 = _loop_attention(q[0, 0], k[0, 0], v[0, 0], 1.1, lambda i, j: True)
    _close(o[0, 0], o2, 1e-13, "O"); _close(lse[0, 0], lse2, 1e-13, "LSE")


def pin_gqa_is_repeated_heads(ex):
    """Query head h reads KV head h // group: the same as repeating each KV
    head group times (and running the plain definition)."""
    r = _rng(6)
    B, hq, hkv, N, d = 2, 8, 2, 15, 4
    q = r.standard_normal((B, hq, N, d)); k = r.standard_normal((B, hkv, N, d)); v = r.standard_normal((B, hkv, N, d))
    for causal in (False, True):
        o, lse = ex(q, k, v, 0.6, causal, 0, 0)
        kr, vr = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
        o2, lse2 = attention_ref(q, kr, vr, 0.6, causal)
        _close(o, o2, 1e-13, "O"); _close(lse, lse2, 1e-13, "LSE")


def pin_cross_attention(ex):
    """Without the causal mask every query sees all S keys, against loops."""
    r = _rng(7)
    T, S, d = 5, 11, 3
    q = r.standard_normal((1, 1, T, d)); k = r.standard_normal((1, 1, S, d)); v = r.standard_normal((1, 1, S, d))
    o, lse = ex(q, k, v, 0.8, False, None, 0)
    o2, lse2 = _loop_attention(q[0, 0], k[0, 0], v[0, 0], 0.8, lambda i, j: True)
    _close(o[0, 0], o2, 1e-13, "O"); _close(lse[0, 0], lse2, 1e-13, "LSE")


PINS = [pin_square_reduces_to_plain, pin_window_one, pin_window_brute_force, pin_chunked_prefill,
        pin_decode_row, pin_gqa_is_repeated_heads, pin_cross_attention]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_variants_oracle_pin(pin):
    pin(attention_ex_ref)


# ------------------------------------------------------------- mutants
def _mutant(kind):
    def ex(q, k, v, scale, causal, offset=None, window=0):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, hq, T, d = q.shape
        hkv, S = k.shape[1], k.shape[2]
        if offset is None:
            offset = 0 if kind == "default_offset_zero" else S - T
        pos = offset + np.arange(T)[:, None]
        j = np.arange(S)[None, :]
        vis = np.ones((T, S), dtype=bool)
        if causal:
            vis &= (j < pos) | (j == pos) if kind != "strict_diagonal" else j < pos
            if window:
                lo = pos - window if kind == "window_off_by_one" else pos - window + 1
                vis &= j >= lo
        o = np.empty((B, hq, T, v.shape[-1])); lse = np.empty((B, hq, T))
        group = hq // hkv
        for b in range(B):
            for h in range(hq):
                kvh = h % hkv if kind == "gqa_modulo" else h // group
                s = np.where(vis, scale * (q[b, h] @ k[b, kvh].T), -np.inf)
                m = s.max(axis=1)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(s - m[:, None])
                l = e.sum(axis=1)
                o[b, h] = (e / np.maximum(l, 1e-300)[:, None]) @ v[b, kvh]
                lse[b, h] = m + np.log(np.maximum(l, 1e-300))
        return o, lse
    return ex


@pytest.mark.parametrize("kind", ["default_offset_zero", "strict_diagonal", "window_off_by_one", "gqa_modulo"])
def test_variants_mutant_is_caught(kind):
    caught = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {kind} passed every pin"


def test_rows_form_matches():
    r = _rng(8)
    T, S, d = 20, 50, 6
    q = r.standard_normal((1, 1, T, d)); k = r.standard_normal((1, 1, S, d)); v = r.standard_normal((1, 1, S, d))
    rows = np.array([0, 3, 19])
    for causal, off, W in ((False, None, 0), (True, None, 0), (True, 10, 7), (True, 30, 1)):
        o, lse = attention_ex_ref(q, k, v, 0.3, causal, off, W)
        o2, lse2 = attention_ex_rows_ref(q[0, 0], k[0, 0], v[0, 0], 0.3, causal, off, W, rows)
        _close(o2, o[0, 0, rows], 1e-13, "O"); _close(lse2, lse[0, 0, rows], 1e-13, "LSE")


def test_argument_errors():
    q = np.zeros((1, 3, 4, 2)); k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        attention_ex_ref(q, k, k, 1.0, False)          # 3 query heads over 2 KV heads
    q = np.zeros((1, 1, 4, 2)); k = np.zeros((1, 1, 6, 2))
    with pytest.raises(ValueError):
        attention_ex_ref(q, k, k, 1.0, False, None, 3)  # window without the causal mask
    with pytest.raises(ValueError):
        attention_ex_ref(q, k, k, 1.0, True, 3, 0)      # offset > S - T


# ------------------------------------------------------------ split-KV merge
from oracle.variants import attention_split_ref, merge_mla_ref, merge_partials_ref  # noqa: E402


@pytest.mark.parametrize("causal,off,W,chunk", [(False, None, 0, 7), (True, None, 0, 5), (True, 10, 6, 4),
                                                (True, 0, 0, 64), (True, None, 3, 1)])
def test_merge_of_partials_equals_unsplit(causal, off, W, chunk):
    """Chunked partials merged == the unsplit definition ("15. FlashAttention",
    "Decode is different: flash-decoding")."""
    r = _rng(40)
    B, hq, hkv, T, S, d = 1, 4, 2, 9, 30, 5
    q = r.standard_normal((B, hq, T, d)); k = r.standard_normal((B, hkv, S, d)); v = r.standard_normal((B, hkv, S, d))
    op, lp = attention_split_ref(q, k, v, 0.7, causal, off, W, chunk)
    o, lse = merge_partials_ref(op, lp)
    o2, lse2 = attention_ex_ref(q, k, v, 0.7, causal, off, W)
    _close(o, o2, 1e-13, "O"); _close(lse, lse2, 1e-13, "LSE")


def test_merge_is_associative_and_matches_the_m_l_a_form():
    """Any grouping of the partials gives the same result, and the (O, L)
    form equals the pages' (m, l, a) form."""
    r = _rng(41)
    G, n, d = 5, 6, 3
    m = r.standard_normal((G, n)) * 3
    l = np.exp(r.standard_normal((G, n)))
    a = r.standard_normal((G, n, d)) * l[..., None]
    o_parts, lse_parts = a / l[..., None], m + np.log(l)
    o, lse = merge_partials_ref(o_parts, lse_parts)
    o2, lse2 = merge_mla_ref([(m[g], l[g], a[g]) for g in range(G)])
    _close(o, o2, 1e-13, "O vs (m, l, a)"); _close(lse, lse2, 1e-13, "LSE vs (m, l, a)")
    oa, la = merge_partials_ref(o_parts[:2], lse_parts[:2])
    ob, lb = merge_partials_ref(o_parts[2:], lse_parts[2:])
    o3, lse3 = merge_partials_ref(np.stack([oa, ob]), np.stack([la, lb]))
    _close(o3, o, 1e-13, "grouped O"); _close(lse3, lse, 1e-13, "grouped LSE")


def test_empty_chunk_contributes_nothing():
    r = _rng(42)
    o_parts = r.standard_normal((3, 4, 2)); lse_parts = r.standard_normal((3, 4))
    lse_parts[1] = -np.inf
    o_parts[1] = np.nan  # never read
    o, lse = merge_partials_ref(o_parts, lse_parts)
    o2, lse2 = merge_partials_ref(o_parts[[0, 2]], lse_parts[[0, 2]])
    _close(o, o2, 1e-15, "O"); _close(lse, lse2, 1e-15, "LSE")
