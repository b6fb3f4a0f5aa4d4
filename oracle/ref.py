"""Plain fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library and never imports it.

What it computes is the plain definition of attention, written out with the
whole score matrix materialised, one (batch, head) at a time:

    S = scale * Q K^T                       (N x N)
    S[i, j] = -inf  where j > i             (only when causal)
    m_i  = max_j S[i, j]
    l_i  = sum_j exp(S[i, j] - m_i)
    P    = exp(S - m) / l                   (row-stochastic)
    O    = P V
    LSE_i = m_i + ln(l_i)  = logsumexp_j S[i, j]

Sources (the pages this follows):
  * "15. FlashAttention" (inference.shantanugoel.com), section "The score
    matrix is the problem": S = QK^T / sqrt(d), P = softmax(S), O = PV.
  * "FlashAttention：从 IO-Aware Attention 到 GPU Work Partitioning"
    (blog.euler0525.cn), sections "Attention 的性能瓶颈" (the three-step
    definition) and "Online Softmax" (the max-subtracted stable softmax,
    m = max s, l = sum e^{s-m}, p = e^{s-m}/l), and section "减少 Non-Matmul
    FLOPs" (L = m + log l is the row logsumexp).
  * "Lecture 3 — FlashAttention-1 Algorithm" (jared-hpc.com), section "The
    forward loop": the kernel writes O and LSE = m + log(l).
  * "15. FlashAttention", sections "The algorithm in plain PyTorch" (a row
    with no visible key is an error) and "The kernel" (the causal rule:
    key position <= query position).

Readings taken where the pages leave a choice open:
  * ``scale`` is an explicit argument (the pages use 1/sqrt(d)); LSE is the
    logsumexp of the *scaled* scores, in natural log.
  * Causal masking is square self-attention: key j is visible to query i
    iff j <= i.
  * Inputs of any float dtype are converted exactly to float64 first; the
    bf16 values the GPU receives are therefore the values the oracle uses.
"""

import numpy as np

__all__ = [
    "as_f64",
    "scores_ref",
    "probabilities_ref",
    "attention_ref",
    "attention_rows_ref",
]


def as_f64(x):
    """Exact conversion of a numpy array (or anything numpy accepts) to float64."""
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def _check_qkv(q, k, v):
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have one shape (square self-attention)")
    if q.ndim < 2:
        raise ValueError("q, k and v need at least the [N, d] axes")


def scores_ref(q, k, scale, causal):
    """Scaled, masked score matrix of one head: q, k are [N, d]; returns [N, N].

    Masked positions hold -inf, so that they contribute exactly exp(-inf) = 0.
    """
    q = as_f64(q)
    k = as_f64(k)
    s = (q @ k.T) * float(scale)
    if causal:
        n = s.shape[0]
        future = np.triu(np.ones((n, n), dtype=bool), k=1)  # j > i
        s = np.where(future, -np.inf, s)
    return s


def probabilities_ref(q, k, scale, causal):
    """P = softmax(S) row by row (max-subtracted), plus m, l and LSE per row."""
    s = scores_ref(q, k, scale, causal)
    m = s.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m[:, None])  # exp(-inf) = 0 exactly at masked positions
    l = e.sum(axis=1)
    p = e / l[:, None]
    lse = m + np.log(l)
    return p, m, l, lse


def attention_ref(q, k, v, scale, causal):
    """O and LSE for [..., N, d] inputs (leading axes are batch, heads, ...).

    Returns (O float64 [..., N, d], LSE float64 [..., N]).
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    _check_qkv(q, k, v)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf = q.reshape(-1, n, d)
    kf = k.reshape(-1, n, d)
    vf = v.reshape(-1, n, d)
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2], dtype=np.float64)
    for g in range(qf.shape[0]):
        if n == 0:
            continue
        p, _, _, lse_g = probabilities_ref(qf[g], kf[g], scale, causal)
        o[g] = p @ vf[g]
        lse[g] = lse_g
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)


def attention_rows_ref(q, k, v, scale, causal, rows):
    """O and LSE of selected query rows of one head, each computed on its own.

    q, k, v are [N, d] arrays of one (batch, head); ``rows`` are query
    indices.  Row i uses keys 0..i when causal, all keys otherwise, exactly as
    the full definition does; no other row is computed.  Used to check large
    problems on a sample of their outputs.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    _check_qkv(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, q.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for r, i in enumerate(rows):
        last = int(i) + 1 if causal else k.shape[0]
        s = (k[:last] @ q[i]) * float(scale)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[r] = (e / l) @ v[:last]
        lse[r] = m + np.log(l)
    return o, lse
