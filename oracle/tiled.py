"""fp64 tiled online-softmax recurrence (Q-outer, KV-inner), for the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/ref.py``): never imported by the
product path, and it shares no code with the HIP library.

This is the algorithm the GPU kernel runs, written as plainly as possible in
float64, so that the tests can show that the recurrence reaches the plain
definition in ``ref.py`` for any tile sizes (B_r, B_c), including tiles that
do not divide N.  Steps, in the pages' order and notation:

  for each query tile Q_i (B_r rows):                  outer loop
      m = -inf, l = 0, acc = 0                         per row
      for each key/value tile K_j, V_j (B_c rows):     inner loop
          S    = scale * Q_i K_j^T                     (masked: -inf)
          m_new = max(m, rowmax S)
          ref   = m_new, or 0 where m_new = -inf       safe reference
          alpha = exp(m - ref)                         rescale of old terms
          P     = exp(S - ref)
          l     = alpha * l + rowsum P
          acc   = alpha * acc + P V_j                  unnormalised output
          m     = m_new
      O_i = acc / l;  LSE_i = m + ln l                 written once

Sources:
  * "Lecture 3 — FlashAttention-1 Algorithm" (jared-hpc.com), section "The
    forward loop (Algorithm 1 from the FA1 paper)": the Q-outer / KV-inner
    loop, running m and l, O and LSE written once per query tile.
  * "15. FlashAttention" (inference.shantanugoel.com), section "Online
    softmax: normalize as you go" (the update of m, p, l, a and O = a / l)
    and section "The algorithm in plain PyTorch" (the safe reference of 0
    for a row that has seen no visible key yet, and the error for a row that
    never sees one).
  * "FlashAttention V1" (infra.bea.ai), section "2. Two Key Techniques"
    (tiling Q into B_r rows and K/V into B_c rows).
  * "FlashAttention：从 IO-Aware Attention 到 GPU Work Partitioning"
    (blog.euler0525.cn), section "减少 Non-Matmul FLOPs": the accumulator is
    kept unnormalised and divided by l once at the end.

The pages write p either as exp(S - m_tile) followed by a second rescale, or
directly as exp(S - m_new); the two are equal in exact arithmetic and this
follows the direct form.
"""

import numpy as np

__all__ = ["tiled_ref"]


def _tiled_head(q, k, v, scale, causal, Br, Bc, trace):
    n, d = q.shape
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    for i0 in range(0, n, Br):                       # query tile Q_i
        i1 = min(n, i0 + Br)
        qi = q[i0:i1]
        qpos = np.arange(i0, i1)
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, d))
        for j0 in range(0, n, Bc):                   # key/value tile K_j, V_j
            j1 = min(n, j0 + Bc)
            s = (qi @ k[j0:j1].T) * float(scale)
            if causal:
                kpos = np.arange(j0, j1)
                s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.exp(m - ref)
            p = np.exp(s - ref[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j1]
            if trace is not None:
                trace.append({
                    "i0": i0, "j0": j0, "m": m_new.copy(), "alpha": alpha.copy(),
                    "p": p.copy(), "l": l.copy(), "a": acc.copy(),
                })
            m = m_new
        if np.any(l == 0):
            raise ValueError("a query row has no visible key")
        o[i0:i1] = acc / l[:, None]
        lse[i0:i1] = m + np.log(l)
    return o, lse


def tiled_ref(q, k, v, scale, causal, Br, Bc, trace=None):
    """Tiled recurrence over [..., N, d] inputs; returns (O, LSE) in float64.

    ``trace``, if a list, receives one dict per (query tile, key tile) step
    with the state after that step (m, alpha, p, l, a); it is only meant for
    small single-head inputs such as the pages' worked example.
    """
    if Br < 1 or Bc < 1:
        raise ValueError("tile sizes must be positive")
    q = np.asarray(q).astype(np.float64)
    k = np.asarray(k).astype(np.float64)
    v = np.asarray(v).astype(np.float64)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have one shape")
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf, kf, vf = (x.reshape(-1, n, d) for x in (q, k, v))
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2])
    for g in range(qf.shape[0]):
        o[g], lse[g] = _tiled_head(qf[g], kf[g], vf[g], scale, causal, int(Br), int(Bc), trace)
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)
