"""Pins that tie the oracle to facts outside itself.

Each ``pin_*`` function takes the implementation under check and raises
AssertionError when it disagrees with what the pages or the mathematics fix:
printed values of the worked example, closed forms, invariants, brute force
on tiny inputs, and one library routine.  ``test_oracle.py`` runs them on the
oracle (all must hold); ``test_oracle_mutants.py`` runs them on copies of the
oracle with a planted mistake (each copy must fail at least one), to show the
pins would catch a plausible error.

``attn(q, k, v, scale, causal) -> (O, LSE)`` works on [..., N, d] arrays.
``tiled(q, k, v, scale, causal, Br, Bc, trace=None) -> (O, LSE)``.
``probs(q, k, scale, causal) -> (P, m, l, LSE)`` for one head.
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def _embed_example(ex):
    """The pages' single row as square attention with d = 1: all four query
    rows are the scalar 1, so row i's scores are exactly the listed scores."""
    s = np.array(ex["scores"], dtype=np.float64)
    vals = np.array(ex["values"], dtype=np.float64)
    n = s.size
    q = np.ones((n, 1))
    k = s.reshape(n, 1)
    v = vals.reshape(n, 1)
    return q, k, v


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- printed values
def pin_worked_example_value(attn):
    """softmax([0,1,2,-1]) . [2,4,1,3] is printed as 1.8619 ("15. FlashAttention",
    section "Worked example")."""
    ex = _load_worked_example()
    q, k, v = _embed_example(ex)
    o, lse = attn(q, k, v, 1.0, False)
    o = np.asarray(o)
    want = ex["printed"]["O"]
    for i in range(o.shape[0]):
        assert round(float(o[i, 0]), ex["decimals"]) == want, (i, o[i, 0], want)


def pin_worked_example_trace(tiled):
    """Every intermediate the page prints for the two-tile walk-through."""
    ex = _load_worked_example()
    q, k, v = _embed_example(ex)
    trace = []
    tiled(q, k, v, 1.0, False, q.shape[0], ex["tile"], trace=trace)
    assert len(trace) == 2, len(trace)
    dec = ex["decimals"]
    t1, t2 = trace[0], trace[1]
    p1 = ex["printed"]["tile1"]
    p2 = ex["printed"]["tile2"]

    def r(x):
        return round(float(x), dec)

    assert r(t1["m"][0]) == p1["m"], t1["m"][0]
    assert [r(x) for x in t1["p"][0]] == p1["p"], t1["p"][0]
    assert r(t1["l"][0]) == p1["l"], t1["l"][0]
    assert r(t1["a"][0, 0]) == p1["a"], t1["a"][0, 0]
    assert r(t2["m"][0]) == p2["m"], t2["m"][0]
    assert r(t2["alpha"][0]) == p2["alpha"], t2["alpha"][0]
    assert [r(x) for x in t2["p"][0]] == p2["p"], t2["p"][0]
    assert r(t2["l"][0]) == p2["l"], t2["l"][0]
    assert r(t2["a"][0, 0]) == p2["a"], t2["a"][0, 0]


# ---------------------------------------------------------------- closed forms
E = math.e
# Row i of the causal worked example sees scores [0, 1, 2, -1][:i+1]:
#   O_i = sum_j e^{s_j} v_j / sum_j e^{s_j},  LSE_i = ln sum_j e^{s_j}.
CAUSAL_EXAMPLE_O = [
    2.0,
    (2.0 + 4.0 * E) / (1.0 + E),
    (2.0 + 4.0 * E + 1.0 * E ** 2) / (1.0 + E + E ** 2),
    (2.0 + 4.0 * E + 1.0 * E ** 2 + 3.0 / E) / (1.0 + E + E ** 2 + 1.0 / E),
]
CAUSAL_EXAMPLE_LSE = [
    0.0,
    math.log(1.0 + E),
    math.log(1.0 + E + E ** 2),
    math.log(1.0 + E + E ** 2 + 1.0 / E),
]


def pin_worked_example_closed_form(attn):
    """Exact values of the worked example, non-causal and causal, and its LSE."""
    ex = _load_worked_example()
    q, k, v = _embed_example(ex)
    o, lse = attn(q, k, v, 1.0, False)
    o, lse = np.asarray(o), np.asarray(lse)
    assert np.allclose(o[:, 0], CAUSAL_EXAMPLE_O[3], rtol=0, atol=1e-13), o[:, 0]
    assert np.allclose(lse, CAUSAL_EXAMPLE_LSE[3], rtol=0, atol=1e-13), lse
    o, lse = attn(q, k, v, 1.0, True)
    o, lse = np.asarray(o), np.asarray(lse)
    assert np.allclose(o[:, 0], CAUSAL_EXAMPLE_O, rtol=0, atol=1e-13), o[:, 0]
    assert np.allclose(lse, CAUSAL_EXAMPLE_LSE, rtol=0, atol=1e-13), lse


def pin_uniform_scores(attn):
    """Q = 0 makes every visible score 0: O_i is the plain mean of the visible
    V rows and LSE_i = ln(#visible) (ln N, or ln(i+1) when causal)."""
    rng = _rng(11)
    n, d = 37, 5
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    o, lse = attn(q, k, v, 0.7, False)
    assert np.allclose(np.asarray(o), np.broadcast_to(v.mean(axis=0), (n, d)), rtol=0, atol=1e-13)
    assert np.allclose(np.asarray(lse), math.log(n), rtol=0, atol=1e-13)
    o, lse = attn(q, k, v, 0.7, True)
    cmean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(np.asarray(o), cmean, rtol=0, atol=1e-13)
    assert np.allclose(np.asarray(lse), np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)


def pin_constant_values(attn):
    """V = c (every row) gives O = c for any Q, K, mask: the weights sum to 1."""
    rng = _rng(12)
    n, d = 29, 6
    q = rng.standard_normal((n, d)) * 3
    k = rng.standard_normal((n, d))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (n, d)).copy()
    for causal in (False, True):
        o, _ = attn(q, k, v, 0.5, causal)
        assert np.allclose(np.asarray(o), v, rtol=0, atol=1e-12), causal


def pin_single_key(attn):
    """N = 1: O = V_0 and LSE = scale * q_0 . k_0."""
    rng = _rng(13)
    d = 7
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    v = rng.standard_normal((1, d))
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.3, causal)
        assert np.allclose(np.asarray(o), v, rtol=0, atol=1e-15)
        assert abs(float(np.asarray(lse).ravel()[0]) - 0.3 * float(q[0] @ k[0])) < 1e-14


# ---------------------------------------------------------------- invariants
def pin_row_stochastic(probs):
    """Rows of P are probability vectors; masked entries are exactly 0; and
    sum_j exp(S_ij - LSE_i) = 1 (LSE is the row logsumexp)."""
    rng = _rng(14)
    n, d = 50, 8
    q = rng.standard_normal((n, d)) * 2
    k = rng.standard_normal((n, d))
    for causal in (False, True):
        p, m, l, lse = probs(q, k, 0.35, causal)
        p = np.asarray(p)
        assert np.all(p >= 0)
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        s = (q @ k.T) * 0.35
        if causal:
            assert np.all(p[np.triu_indices(n, 1)] == 0.0)
            s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
        assert np.allclose(np.exp(s - np.asarray(lse)[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-13)


def pin_shift_invariance(attn):
    """K' = K + 1 u^T adds scale * q_i . u to every score of row i: O is
    unchanged and LSE_i grows by exactly that amount (causal or not)."""
    rng = _rng(15)
    n, d = 33, 4
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    u = rng.standard_normal(d)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, 0.8, causal)
        o2, l2 = attn(q, k + u[None, :], v, 0.8, causal)
        assert np.allclose(np.asarray(o1), np.asarray(o2), rtol=0, atol=1e-12)
        assert np.allclose(np.asarray(l2) - np.asarray(l1), 0.8 * (q @ u), rtol=0, atol=1e-12)


def pin_permutation(attn):
    """Non-causal: permuting K and V rows together changes nothing; permuting
    Q rows permutes O and LSE the same way."""
    rng = _rng(16)
    n, d = 31, 6
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    o, lse = attn(q, k, v, 0.4, False)
    pk = rng.permutation(n)
    o2, lse2 = attn(q, k[pk], v[pk], 0.4, False)
    assert np.allclose(np.asarray(o), np.asarray(o2), rtol=0, atol=1e-12)
    assert np.allclose(np.asarray(lse), np.asarray(lse2), rtol=0, atol=1e-12)
    pq = rng.permutation(n)
    o3, lse3 = attn(q[pq], k, v, 0.4, False)
    assert np.allclose(np.asarray(o)[pq], np.asarray(o3), rtol=0, atol=1e-12)
    assert np.allclose(np.asarray(lse)[pq], np.asarray(lse3), rtol=0, atol=1e-12)


def pin_large_scores(attn):
    """Scores in the thousands must not overflow: compared with the same
    brute force as below, which subtracts the row max in exact sums."""
    rng = _rng(17)
    n, d = 9, 3
    q = rng.standard_normal((n, d)) * 60
    k = rng.standard_normal((n, d)) * 60
    v = rng.standard_normal((n, d))
    for causal in (False, True):
        o, lse = attn(q, k, v, 1.0, causal)
        ob, lb = _brute(q, k, v, 1.0, causal)
        assert np.all(np.isfinite(np.asarray(o)))
        assert np.allclose(np.asarray(o), ob, rtol=0, atol=1e-12)
        assert np.allclose(np.asarray(lse), lb, rtol=1e-14, atol=1e-11)


# ---------------------------------------------------------------- brute force
def _brute(q, k, v, scale, causal):
    """Scalar loops with math.exp and math.fsum, one score at a time."""
    n, d = q.shape
    o = np.zeros((n, d))
    lse = np.zeros(n)
    for i in range(n):
        visible = range(i + 1) if causal else range(n)
        sc = [scale * math.fsum(float(q[i, t]) * float(k[j, t]) for t in range(d)) for j in visible]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = math.fsum(w)
        for t in range(d):
            o[i, t] = math.fsum(wj * float(v[j, t]) for wj, j in zip(w, visible)) / tot
        lse[i] = mx + math.log(tot)
    return o, lse


def pin_brute_force(attn):
    """N <= 16, d in {1, 2, 3, 8}, both masks, against scalar brute force."""
    rng = _rng(18)
    for n in (1, 2, 5, 16):
        for d in (1, 2, 3, 8):
            q = rng.standard_normal((n, d))
            k = rng.standard_normal((n, d))
            v = rng.standard_normal((n, d))
            scale = 1.0 / math.sqrt(d)
            for causal in (False, True):
                o, lse = attn(q, k, v, scale, causal)
                ob, lb = _brute(q, k, v, scale, causal)
                assert np.allclose(np.asarray(o), ob, rtol=0, atol=1e-13), (n, d, causal)
                assert np.allclose(np.asarray(lse), lb, rtol=0, atol=1e-13), (n, d, causal)


def pin_library_sdpa(attn):
    """torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine; it checks the oracle only, never the GPU path)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(19)
    B, H, n, d = 2, 3, 45, 16
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    for causal in (False, True):
        o, _ = attn(q, k, v, 0.25, causal)
        ot = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.25).numpy()
        assert np.allclose(np.asarray(o), ot, rtol=0, atol=1e-12), causal


def pin_tiled_matches(attn, tiled, quick=False):
    """The recurrence reaches the definition for any tile sizes, including
    ones that do not divide N (invariant of the online softmax)."""
    rng = _rng(20)
    cases = [(1, 3), (5, 4), (64, 8), (100, 8)]
    if not quick:
        cases.append((1000, 16))
    for n, d in cases:
        q = rng.standard_normal((n, d)) * 1.5
        k = rng.standard_normal((n, d)) * 1.5
        v = rng.standard_normal((n, d))
        sizes = [1, 2, 3, 7, 16, 64, 128, n]
        if n >= 1000:
            sizes = [7, 64, 128, n]          # small tiles at N = 1000 take minutes in Python
        for causal in (False, True):
            o, lse = attn(q, k, v, 0.3, causal)
            o, lse = np.asarray(o), np.asarray(lse)
            for Br in sizes:
                for Bc in sizes:
                    if Br > n and Br != n or Bc > n and Bc != n:
                        continue
                    ot, lt = tiled(q, k, v, 0.3, causal, Br, Bc)
                    assert np.allclose(ot, o, rtol=1e-12, atol=1e-12), (n, Br, Bc, causal)
                    assert np.allclose(lt, lse, rtol=1e-12, atol=1e-12), (n, Br, Bc, causal)
