"""Pins that tie the backward oracle to facts outside itself.

Each ``pin_*`` function takes the implementation under check,
``bwd(q, k, v, do, scale, causal) -> (dQ, dK, dV, D)`` on [N, d] arrays, and
raises AssertionError when it disagrees with what the mathematics fixes:
central finite differences of a forward written out here with scalar loops,
fp64 autograd of the textbook attention in torch, closed forms and
invariants.  ``test_oracle_bwd.py`` runs them on the oracle (all must hold)
and on copies of it with a planted mistake (each copy must fail one).
"""

import math

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def _loop_forward(q, k, v, scale, causal):
    """O of square attention with scalar loops and math.fsum (tiny N only)."""
    n, d = q.shape
    dv = v.shape[1]
    o = np.zeros((n, dv))
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = [scale * math.fsum(q[i, e] * k[j, e] for e in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        for c in range(dv):
            o[i, c] = math.fsum(wj * v[j, c] for wj, j in zip(w, keys)) / tot
    return o


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    bound = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= bound, f"{what}: max err {err:.3e} > {bound:.3e}"


# ------------------------------------------------------------ finite differences
def pin_bwd_finite_differences(bwd):
    """Gradients of L = sum(O * G) against central differences of a forward
    written out with scalar loops (h = 1e-5, truncation error ~ h^2)."""
    h = 1e-5
    for seed, (n, d, causal) in enumerate([(1, 2, False), (3, 2, True), (4, 3, False), (5, 2, True)]):
        r = _rng(100 + seed)
        q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
        scale = 0.7
        dq, dk, dv, _ = bwd(q, k, v, g, scale, causal)
        for name, x, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
                args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
                lp = float(np.sum(_loop_forward(*args_p, scale, causal) * g))
                lm = float(np.sum(_loop_forward(*args_m, scale, causal) * g))
                num[idx] = (lp - lm) / (2 * h)
            _close(grad, num, atol=1e-7, what=f"{name} n={n} d={d} causal={causal}")


# ------------------------------------------------------------------ library
def pin_bwd_autograd(bwd):
    """fp64 autograd (CPU) of the textbook attention softmax(scale Q K^T + mask) V."""
    for seed, (n, d, causal) in enumerate([(7, 4, False), (9, 5, True), (16, 8, True)]):
        r = _rng(200 + seed)
        q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = scale * (tq @ tk.T)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        (o * torch.tensor(g)).sum().backward()
        dq, dk, dv, _ = bwd(q, k, v, g, scale, causal)
        _close(dq, tq.grad.numpy(), atol=1e-12, rtol=1e-12, what="dQ")
        _close(dk, tk.grad.numpy(), atol=1e-12, rtol=1e-12, what="dK")
        _close(dv, tv.grad.numpy(), atol=1e-12, rtol=1e-12, what="dV")


# ------------------------------------------------------------- closed forms
def pin_bwd_single_key(bwd):
    """N = 1: P = 1, so O = V_0 and dV = dO, while dQ = dK = 0."""
    r = _rng(300)
    q, k, v, g = (r.standard_normal((1, 6)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv, _ = bwd(q, k, v, g, 0.5, causal)
        _close(dv, g, atol=1e-15, what="dV")
        _close(dq, 0 * q, atol=1e-15, what="dQ")
        _close(dk, 0 * k, atol=1e-15, what="dK")


def pin_bwd_constant_values(bwd):
    """All V rows equal: O does not depend on the scores, so dQ = dK = 0."""
    r = _rng(301)
    n, d = 11, 5
    q, k, g = (r.standard_normal((n, d)) for _ in range(3))
    v = np.tile(r.standard_normal((1, d)), (n, 1))
    for causal in (False, True):
        dq, dk, _, _ = bwd(q, k, v, g, 0.8, causal)
        _close(dq, 0 * q, atol=1e-13, what="dQ")
        _close(dk, 0 * k, atol=1e-13, what="dK")


def pin_bwd_uniform_scores(bwd):
    """Q = 0: every visible key has weight 1/n_i, so dK = scale dS^T Q = 0 and
    dV_j = sum over the queries i that see j of dO_i / n_i."""
    r = _rng(302)
    n, d = 9, 4
    k, v, g = (r.standard_normal((n, d)) for _ in range(3))
    q = np.zeros((n, d))
    for causal in (False, True):
        _, dk, dv, _ = bwd(q, k, v, g, 0.9, causal)
        want = np.zeros((n, d))
        for i in range(n):
            vis = range(i + 1) if causal else range(n)
            for j in vis:
                want[j] += g[i] / len(vis)
        _close(dv, want, atol=1e-14, what="dV")
        _close(dk, 0 * k, atol=1e-15, what="dK")


# --------------------------------------------------------------- invariants
def pin_bwd_key_shift(bwd):
    """Adding one vector u to every key adds scale q_i . u to the whole of row
    i, which softmax ignores: the sum over keys of dK is 0 (any mask)."""
    r = _rng(303)
    n, d = 13, 6
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        _, dk, _, _ = bwd(q, k, v, g, 0.6, causal)
        _close(dk.sum(axis=0), np.zeros(d), atol=1e-13, what="sum dK")


def pin_bwd_dv_total(bwd):
    """Rows of P sum to 1, so the sum over keys of dV is the sum over queries
    of dO."""
    r = _rng(304)
    n, d = 12, 5
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        _, _, dv, _ = bwd(q, k, v, g, 0.6, causal)
        _close(dv.sum(axis=0), g.sum(axis=0), atol=1e-13, what="sum dV")


def pin_bwd_delta_is_o_dot_do(bwd):
    """D_i, the row sum of P * dP, equals O_i . dO_i (O from the scalar-loop
    forward)."""
    r = _rng(305)
    n, d = 8, 3
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        _, _, _, delta = bwd(q, k, v, g, 0.75, causal)
        o = _loop_forward(q, k, v, 0.75, causal)
        _close(delta, np.sum(o * g, axis=1), atol=1e-13, what="D")


def pin_bwd_permutation(bwd):
    """Non-causal: permuting the rows of K and V together permutes dK and dV
    the same way and leaves dQ unchanged."""
    r = _rng(306)
    n, d = 10, 4
    q, k, v, g = (r.standard_normal((n, d)) for _ in range(4))
    perm = r.permutation(n)
    dq, dk, dv, _ = bwd(q, k, v, g, 0.5, False)
    dq2, dk2, dv2, _ = bwd(q, k[perm], v[perm], g, 0.5, False)
    _close(dq2, dq, atol=1e-13, what="dQ")
    _close(dk2, dk[perm], atol=1e-13, what="dK")
    _close(dv2, dv[perm], atol=1e-13, what="dV")


BWD_PINS = [
    pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_single_key, pin_bwd_constant_values,
    pin_bwd_uniform_scores, pin_bwd_key_shift, pin_bwd_dv_total, pin_bwd_delta_is_o_dot_do,
    pin_bwd_permutation,
]
