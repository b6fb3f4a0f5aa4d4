"""The split-KV oracle (per-chunk partials and their log-sum-exp merge)
against planted mistakes: each copy of the merge or of the chunking with
one plausible mistake must fail at least one of the pins below, which tie
the pair to facts outside it ("15. FlashAttention", section "Decode is
different: flash-decoding": the merged partials equal the unsplit
attention; the (m, l, a) merge rule; any grouping of the partials; a chunk
the row sees nothing of contributes nothing)."""

import numpy as np
import pytest

from oracle.variants import attention_ex_ref, attention_split_ref, merge_mla_ref, merge_partials_ref


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: max err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ pins
# Each pin takes (split, merge) with the signatures of attention_split_ref
# and merge_partials_ref.  attention_ex_ref is pinned on its own
# (test_oracle_variants.py), merge_mla_ref is the pages' (m, l, a) rule
# written out separately.

def pin_merge_equals_unsplit(split, merge):
    r = _rng(60)
    B, hq, hkv, T, S, d = 1, 4, 2, 9, 30, 5
    q = r.standard_normal((B, hq, T, d))
    k = r.standard_normal((B, hkv, S, d))
    v = r.standard_normal((B, hkv, S, d))
    for causal, off, W, chunk in ((False, None, 0, 7), (True, None, 0, 5), (True, 10, 6, 4), (True, None, 3, 1)):
        op, lp = split(q, k, v, 0.7, causal, off, W, chunk)
        o, lse = merge(op, lp)
        o2, lse2 = attention_ex_ref(q, k, v, 0.7, causal, off, W)
        _close(o, o2, 1e-12, f"O causal={causal} chunk={chunk}")
        _close(lse, lse2, 1e-12, f"LSE causal={causal} chunk={chunk}")


def pin_merge_is_the_m_l_a_rule(split, merge):
    r = _rng(61)
    G, n, d = 5, 6, 3
    m = r.standard_normal((G, n)) * 3
    l = np.exp(r.standard_normal((G, n)))
    a = r.standard_normal((G, n, d)) * l[..., None]
    o, lse = merge(a / l[..., None], m + np.log(l))
    o2, lse2 = merge_mla_ref([(m[g], l[g], a[g]) for g in range(G)])
    _close(o, o2, 1e-12, "O vs (m, l, a)")
    _close(lse, lse2, 1e-12, "LSE vs (m, l, a)")


def pin_merge_grouping(split, merge):
    r = _rng(62)
    op = r.standard_normal((6, 4, 3))
    lp = r.standard_normal((6, 4)) * 5
    o, lse = merge(op, lp)
    oa, la = merge(op[:2], lp[:2])
    ob, lb = merge(op[2:], lp[2:])
    o3, lse3 = merge(np.stack([oa, ob]), np.stack([la, lb]))
    _close(o3, o, 1e-12, "grouped O")
    _close(lse3, lse, 1e-12, "grouped LSE")


def pin_empty_partial(split, merge):
    r = _rng(63)
    op = r.standard_normal((3, 4, 2))
    lp = r.standard_normal((3, 4))
    lp[1] = -np.inf
    op[1] = np.nan  # an empty chunk's O is never read
    o, lse = merge(op, lp)
    o2, lse2 = merge(op[[0, 2]], lp[[0, 2]])
    _close(o, o2, 1e-15, "O")
    _close(lse, lse2, 1e-15, "LSE")


def pin_large_partials_stay_finite(split, merge):
    """Partials whose L_g are near +-1e4 (scores of that size) merge to a
    finite result equal to the shifted closed form."""
    lp = np.array([[1.0e4], [1.0e4 - 1.0], [-1.0e4]])
    op = np.array([[[1.0]], [[3.0]], [[5.0]]])
    o, lse = merge(op, lp)
    w = np.array([1.0, np.exp(-1.0), 0.0])
    _close(o, [[(w @ op[:, 0, 0]) / w.sum()]], 1e-12, "O")
    _close(lse, [1.0e4 + np.log(w.sum())], 1e-9, "LSE")


PINS = [pin_merge_equals_unsplit, pin_merge_is_the_m_l_a_rule, pin_merge_grouping, pin_empty_partial,
        pin_large_partials_stay_finite]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_split_oracle_pin(pin):
    pin(attention_split_ref, merge_partials_ref)


# --------------------------------------------------------------- mutants
def _merge_mutant(kind):
    def merge(o_parts, lse_parts):
        o_parts = np.asarray(o_parts, dtype=np.float64)
        lse_parts = np.asarray(lse_parts, dtype=np.float64)
        m = lse_parts.max(axis=0)
        if kind == "no_max_shift":
            w = np.exp(lse_parts)
            tot = w.sum(axis=0)
            o = np.einsum("g...,g...d->...d", w, np.where(np.isfinite(lse_parts)[..., None], o_parts, 0.0))
            return o / tot[..., None], np.log(tot)
        w = np.exp(lse_parts - m[None])
        tot = w.sum(axis=0)
        keep = np.isfinite(lse_parts)[..., None]
        src = o_parts if kind == "empty_not_skipped" else np.where(keep, o_parts, 0.0)
        o = np.einsum("g...,g...d->...d", w, src)
        if kind != "no_normalise":
            o = o / tot[..., None]
        if kind == "lse_is_max":
            lse = m
        elif kind == "lse_base2":
            lse = m + np.log2(tot)
        else:
            lse = m + np.log(tot)
        return o, lse
    return merge


def _split_mutant(kind):
    """The partials written out again with one mistake: chunk g also takes
    the first key of chunk g + 1 (overlapping_chunks), or L_g is the
    chunk's row max m_g instead of m_g + ln l_g (partial_lse_without_log_l)."""
    from oracle.variants import visible_mask

    def split(q, k, v, scale, causal, offset=None, window=0, chunk=None):
        B, hq, T, d = q.shape
        hkv, S = k.shape[1], k.shape[2]
        off = S - T if offset is None else offset
        vis = visible_mask(T, S, causal, off, window)
        G = -(-S // chunk)
        group = hq // hkv
        o = np.zeros((G, B, hq, T, v.shape[-1]))
        lse = np.full((G, B, hq, T), -np.inf)
        for g in range(G):
            c1 = min(S, (g + 1) * chunk + (1 if kind == "overlapping_chunks" else 0))
            vg = np.zeros_like(vis)
            vg[:, g * chunk:c1] = vis[:, g * chunk:c1]
            rows = vg.any(axis=1)
            if not rows.any():
                continue
            for b in range(B):
                for h in range(hq):
                    s = np.where(vg, scale * (q[b, h] @ k[b, h // group].T), -np.inf)[rows]
                    mx = s.max(axis=1)
                    e = np.exp(s - mx[:, None])
                    o[g, b, h, rows] = (e / e.sum(axis=1)[:, None]) @ v[b, h // group]
                    lse[g, b, h, rows] = mx if kind == "partial_lse_without_log_l" else mx + np.log(e.sum(axis=1))
        return o, lse
    return split


MERGE_MUTANTS = ["no_max_shift", "empty_not_skipped", "no_normalise", "lse_is_max", "lse_base2"]
SPLIT_MUTANTS = ["overlapping_chunks", "partial_lse_without_log_l"]


def _caught(split, merge):
    names = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(split, merge)
        except AssertionError:
            names.append(pin.__name__)
    return names


@pytest.mark.parametrize("kind", MERGE_MUTANTS)
def test_merge_mutant_is_caught(kind):
    assert _caught(attention_split_ref, _merge_mutant(kind)), f"merge mutant {kind} passed every pin"


def test_split_rewrite_without_mistake_passes():
    """The re-implementation the split mutants start from is itself right."""
    assert not _caught(_split_mutant("none"), merge_partials_ref)


@pytest.mark.parametrize("kind", SPLIT_MUTANTS)
def test_split_mutant_is_caught(kind):
    assert _caught(_split_mutant(kind), merge_partials_ref), f"split mutant {kind} passed every pin"
