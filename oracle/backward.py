"""Plain fp64 CPU oracle for the backward pass of exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library and never imports it.

Given the forward O = P V with P = softmax(S), S = scale * Q K^T (causal:
key j visible to query i iff j <= i), and an upstream gradient dO, the
gradients are, written out with every N x N matrix materialised:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij            (equal to O_i . dO_i)
    dS = P * (dP - D)                 (gradient with respect to S)
    dQ = scale * dS K
    dK = scale * dS^T Q

Sources (the pages this follows):
  * "FlashAttention：从 IO-Aware Attention 到 GPU Work Partitioning"
    (blog.euler0525.cn), section "Tiling、Fusion 与 Backward Recomputation":
    the five gradient formulas above, D_i as the row sum of P * dP and its
    identity with O_i . dO_i, and recomputing S and P in the backward
    instead of storing P; section "减少 Non-Matmul FLOPs": P is rebuilt from
    the saved row log-sum-exp, P_ij = exp(S_ij - L_i).
  * "FlashAttention V1" (infra.bea.ai), section "5. The Backward Pass":
    scores are recomputed from Q, K, V during the backward.
  * "Lecture 3 — FlashAttention-1 Algorithm" (jared-hpc.com), section
    "Backward in one sentence": the recomputation uses the saved LSE.

Reading taken where the pages leave a choice open: the pages write the
gradients for S = Q K^T without a scale.  With the explicit scale of the
forward (S = scale * Q K^T), dS is the gradient with respect to the scaled
scores and the chain rule puts one factor ``scale`` on dQ and on dK.
"""

import numpy as np

from .ref import as_f64, probabilities_ref


def attention_bwd_ref(q, k, v, do, scale, causal):
    """Gradients (dQ, dK, dV) of sum(O * dO) for one (batch, head): q, k, v
    and do are [N, d]; plus D (the row sums of P * dP), from the plain
    definition: P is the materialised softmax of the scaled, masked
    scores."""
    q, k, v, do = (as_f64(x) for x in (q, k, v, do))
    p, _, _, _ = probabilities_ref(q, k, scale, causal)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    delta = np.sum(p * dp, axis=-1)
    ds = p * (dp - delta[..., None])
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    return dq, dk, dv, delta


def attention_bwd_from_lse_ref(q, k, v, o, lse, do, scale, causal):
    """The same gradients in the recomputation form the pages describe:
    P_ij = exp(S_ij - L_i) from the saved natural-log LSE, and
    D_i = O_i . dO_i from the forward output instead of a row of P * dP."""
    q, k, v, o, lse, do = (as_f64(x) for x in (q, k, v, o, lse, do))
    n = q.shape[-2]
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        future = np.triu(np.ones((n, n), dtype=bool), k=1)
        s = np.where(future, -np.inf, s)
    p = np.exp(s - lse[..., None])
    delta = np.sum(o * do, axis=-1)
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - delta[..., None])
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    return dq, dk, dv, delta


def attention_bwd_rows_ref(q, k, v, do, scale, causal, rows):
    """dQ of the given query rows only, for one (batch, head): row i uses
    keys 0..i when causal.  dQ_i depends only on row i of P and dP, so each
    row is computed on its own from the definition."""
    q, k, v, do = (as_f64(x) for x in (q, k, v, do))
    rows = np.asarray(rows)
    out = np.zeros((rows.size, q.shape[-1]))
    for r, i in enumerate(rows):
        nk = i + 1 if causal else k.shape[0]
        s = scale * (k[:nk] @ q[i])
        p = np.exp(s - s.max())
        p /= p.sum()
        dp = v[:nk] @ do[i]
        ds = p * (dp - np.dot(p, dp))
        out[r] = scale * (ds @ k[:nk])
    return out


def attention_bwd_cols_ref(q, k, v, do, scale, causal, cols, block=512):
    """dK and dV of the given key rows only, for one (batch, head): key j
    receives gradient from every query that sees it (i >= j when causal).
    Each query's softmax row is needed in full, so P, dP and D are formed
    for ``block`` queries at a time from the definition, and only the
    selected columns of dS and P are used."""
    q, k, v, do = (as_f64(x) for x in (q, k, v, do))
    cols = np.asarray(cols)
    n = q.shape[0]
    dk = np.zeros((cols.size, q.shape[-1]))
    dv = np.zeros((cols.size, v.shape[-1]))
    keys = np.arange(n)
    for i0 in range(0, n, block):
        i1 = min(n, i0 + block)
        s = scale * (q[i0:i1] @ k.T)
        if causal:
            s = np.where(keys[None, :] > np.arange(i0, i1)[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = do[i0:i1] @ v.T
        delta = np.sum(p * dp, axis=1)
        ds = p * (dp - delta[:, None])
        dv += p[:, cols].T @ do[i0:i1]
        dk += scale * (ds[:, cols].T @ q[i0:i1])
    return dk, dv
