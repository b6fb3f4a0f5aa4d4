"""Plain fp64 CPU oracle for the attention variants: grouped K/V heads
(GQA), queries at an offset into a longer key sequence (T != S) and a
sliding window.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library and never imports it.

For q [B, Hq, T, d] and k, v [B, Hkv, S, d], query head h attends with KV
head h // (Hq / Hkv); query row i sits at absolute position p_i = offset + i
(default offset = S - T: the queries are the newest positions); key j is
visible to row i iff j < S and, when causal, j <= p_i and, with a window W,
j >= p_i - W + 1.  Then, with the score matrix materialised,
S = scale * q k^T (masked to -inf), O = softmax(S) v and
LSE = logsumexp(S) per row.

Split-KV (flash-decoding): ``attention_split_ref`` computes the partial
result of each key chunk and ``merge_partials_ref`` combines them.

Sources (the pages this follows): "15. FlashAttention"
(inference.shantanugoel.com), section "The kernel" (query head h reads KV
head h // group; query row i at absolute position offset + i with default
offset S - T, serving prefill, chunked prefill and decode; key visible iff
its position is at most the query's and below S), section "The algorithm in
plain PyTorch" (masking by positions; a row with no visible key is an
error), and its stretch list (a sliding window that skips keys before
q_pos - window).

Readings taken where the pages leave a choice open:
  * A window of W covers exactly W keys ending at the diagonal,
    p_i - W + 1 <= j <= p_i; it is defined only together with the causal
    mask.  W = 0 means no window.
  * 0 <= offset <= S - T, so every row sees at least its diagonal key (and
    key 0 without a window): no row is ever empty.
  * Without the causal mask the offset has no effect: every query sees all
    S keys (cross-attention).
"""

import numpy as np

from .ref import as_f64


def visible_mask(T, S, causal, offset=None, window=0):
    """Boolean [T, S]: True where key j is visible to query row i."""
    if offset is None:
        offset = S - T
    pos = offset + np.arange(T)[:, None]
    j = np.arange(S)[None, :]
    vis = np.ones((T, S), dtype=bool)
    if causal:
        vis &= j <= pos
        if window:
            vis &= j >= pos - window + 1
    return vis


def _check(T, S, causal, offset, window, hq, hkv):
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if window < 0 or (window and not causal):
        raise ValueError("a window needs the causal mask and must be >= 1")
    if causal and not 0 <= offset <= S - T:
        raise ValueError("the offset must satisfy 0 <= offset <= S - T")


def attention_ex_ref(q, k, v, scale, causal, offset=None, window=0):
    """O [B, Hq, T, d] and LSE [B, Hq, T] (float64) from the definition."""
    q, k, v = (as_f64(x) for x in (q, k, v))
    B, hq, T, d = q.shape
    hkv, S = k.shape[1], k.shape[2]
    if offset is None:
        offset = S - T
    _check(T, S, causal, offset, window, hq, hkv)
    group = hq // hkv
    vis = visible_mask(T, S, causal, offset, window)
    o = np.empty((B, hq, T, v.shape[-1]))
    lse = np.empty((B, hq, T))
    for b in range(B):
        for h in range(hq):
            kh, vh = k[b, h // group], v[b, h // group]
            s = np.where(vis, scale * (q[b, h] @ kh.T), -np.inf)
            m = s.max(axis=1)
            if not np.all(np.isfinite(m)):
                raise ValueError("a query row has no visible key")
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            o[b, h] = (e / l[:, None]) @ vh
            lse[b, h] = m + np.log(l)
    return o, lse


def attention_ex_rows_ref(q, k, v, scale, causal, offset, window, rows):
    """O and LSE of selected query rows of one head (q [T, d], k, v [S, d]),
    each row from its own visible keys."""
    q, k, v = (as_f64(x) for x in (q, k, v))
    T, S = q.shape[0], k.shape[0]
    if offset is None:
        offset = S - T
    rows = np.asarray(rows)
    o = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    for r, i in enumerate(rows):
        lo, hi = 0, S
        if causal:
            p = offset + int(i)
            hi = min(S, p + 1)
            if window:
                lo = max(0, p - window + 1)
        s = scale * (k[lo:hi] @ q[i])
        m = s.max()
        e = np.exp(s - m)
        o[r] = (e @ v[lo:hi]) / e.sum()
        lse[r] = m + np.log(e.sum())
    return o, lse


def merge_partials_ref(o_parts, lse_parts):
    """Merge partial results of disjoint key chunks: with O_g the softmax
    output over chunk g alone and L_g its log-sum-exp (-inf for a chunk
    with no visible key, whose O_g is ignored),
        L = log sum_g exp(L_g),   O = sum_g exp(L_g - L) O_g.
    ("15. FlashAttention", section "Decode is different: flash-decoding":
    the (m, l, a) merge rule, here in its (O, L) form.)  Arrays are
    [splits, ..., d] and [splits, ...]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m[None])  # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=0)
    o = np.einsum("g...,g...d->...d", w, np.where(np.isfinite(lse_parts)[..., None], o_parts, 0.0))
    return o / tot[..., None], m + np.log(tot)


def merge_mla_ref(parts):
    """The same merge in the pages' (m, l, a) form: m = max m_g,
    l = sum e^{m_g - m} l_g, a = sum e^{m_g - m} a_g, O = a / l.  ``parts``
    is a list of (m [...], l [...], a [..., d])."""
    m = np.max([p[0] for p in parts], axis=0)
    l = sum(np.exp(p[0] - m) * p[1] for p in parts)
    a = sum(np.exp(p[0] - m)[..., None] * p[2] for p in parts)
    return a / l[..., None], m + np.log(l)


def attention_split_ref(q, k, v, scale, causal, offset=None, window=0, chunk=None):
    """Partial (O_g, L_g) of every key chunk of ``chunk`` keys, each from the
    definition over the keys of its chunk that a row sees (O_g = 0 and
    L_g = -inf where it sees none); returns (O_parts [G, B, Hq, T, d],
    LSE_parts [G, B, Hq, T])."""
    q, k, v = (as_f64(x) for x in (q, k, v))
    B, hq, T, d = q.shape
    hkv, S = k.shape[1], k.shape[2]
    if offset is None:
        offset = S - T
    group = hq // hkv
    vis = visible_mask(T, S, causal, offset, window)
    G = -(-S // chunk)
    o = np.zeros((G, B, hq, T, v.shape[-1]))
    lse = np.full((G, B, hq, T), -np.inf)
    for g in range(G):
        c0, c1 = g * chunk, min(S, (g + 1) * chunk)
        vg = vis[:, c0:c1]
        rows = vg.any(axis=1)
        for b in range(B):
            for h in range(hq):
                kh, vh = k[b, h // group, c0:c1], v[b, h // group, c0:c1]
                s = np.where(vg, scale * (q[b, h] @ kh.T), -np.inf)[rows]
                if s.size == 0:
                    continue
                m = s.max(axis=1)
                e = np.exp(s - m[:, None])
                l = e.sum(axis=1)
                o[g, b, h, rows] = (e / l[:, None]) @ vh
                lse[g, b, h, rows] = m + np.log(l)
    return o, lse
