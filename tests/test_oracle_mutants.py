"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant below is the oracle's definition with one plausible error (a
dropped term, a wrong sign or index, a transposed operand, the wrong log
base, ...).  A mutant that passed every pin would show a blind spot of the
pins; the test requires that none does.  The real oracle is never modified.
"""

import math

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention_ref, probabilities_ref, tiled_ref


def _definition(q, k, v, scale, causal, *, no_scale=False, mask="causal", lse_base="e",
                lse_no_max=False, transpose_scores=False, no_max_sub=False, axis=1,
                pt=False):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    n, d = q.shape[-2:]
    qf, kf, vf = (x.reshape(-1, n, d) for x in (q, k, v))
    o = np.empty_like(qf)
    lse = np.empty(qf.shape[:2])
    for g in range(qf.shape[0]):
        s = qf[g] @ kf[g].T
        if transpose_scores:
            s = s.T
        if not no_scale:
            s = s * scale
        if causal:
            if mask == "causal":
                bad = np.triu(np.ones((n, n), bool), 1)
            elif mask == "strict":
                bad = np.triu(np.ones((n, n), bool), 0)
            else:  # anti-causal
                bad = np.tril(np.ones((n, n), bool), -1)
            s = np.where(bad, -np.inf, s)
        m = s.max(axis=axis, keepdims=True)
        if not np.all(np.isfinite(m)):
            raise ValueError("no visible key")
        e = np.exp(s) if no_max_sub else np.exp(s - m)
        l = e.sum(axis=axis, keepdims=True)
        p = e / l
        o[g] = (p.T if pt else p) @ vf[g]
        ll = np.log(l.ravel()) if not no_max_sub else np.log(l.ravel())
        if lse_base == "2":
            ll = np.log2(l.ravel())
        lse[g] = ll if (lse_no_max or no_max_sub) else m.ravel() + ll
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)


def _tiled_mutant(kind):
    """The recurrence with one planted mistake."""
    def tiled(q, k, v, scale, causal, Br, Bc, trace=None):
        q = np.asarray(q, float); k = np.asarray(k, float); v = np.asarray(v, float)
        n, d = q.shape
        o = np.zeros((n, d)); lse = np.zeros(n)
        for i0 in range(0, n, Br):
            i1 = min(n, i0 + Br)
            m = np.full(i1 - i0, -np.inf); l = np.zeros(i1 - i0); acc = np.zeros((i1 - i0, d))
            for j0 in range(0, n, Bc):
                j1 = min(n, j0 + Bc)
                s = q[i0:i1] @ k[j0:j1].T * scale
                if causal:
                    s = np.where(np.arange(j0, j1)[None, :] <= np.arange(i0, i1)[:, None], s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.exp(m - ref)
                if kind == "alpha_inverted":
                    alpha = np.exp(ref - m) if np.all(np.isfinite(m)) else alpha
                p = np.exp(s - ref[:, None])
                l = (l if kind == "no_l_rescale" else alpha * l) + p.sum(axis=1)
                acc = (acc if kind == "no_acc_rescale" else alpha[:, None] * acc) + p @ v[j0:j1]
                if kind == "stale_max":
                    m_new = np.where(np.isfinite(m), m, m_new)
                if trace is not None:
                    trace.append({"m": m_new.copy(), "alpha": alpha.copy(), "p": p.copy(),
                                  "l": l.copy(), "a": acc.copy()})
                m = m_new
            o[i0:i1] = acc / l[:, None]
            lse[i0:i1] = m + np.log(l)
        return o, lse
    return tiled


DEFINITION_MUTANTS = {
    "no_scale": dict(no_scale=True),
    "strict_causal_mask": dict(mask="strict"),
    "anti_causal_mask": dict(mask="anti"),
    "lse_log2": dict(lse_base="2"),
    "lse_without_max": dict(lse_no_max=True),
    "transposed_scores": dict(transpose_scores=True),
    "no_max_subtraction": dict(no_max_sub=True),
    "softmax_over_columns": dict(axis=0),
    "p_transposed_in_pv": dict(pt=True),
}

DEFINITION_PINS = [
    pins.pin_worked_example_value, pins.pin_worked_example_closed_form, pins.pin_uniform_scores,
    pins.pin_constant_values, pins.pin_single_key, pins.pin_shift_invariance,
    pins.pin_permutation, pins.pin_large_scores, pins.pin_brute_force, pins.pin_library_sdpa,
]


def _fails(pin, *args):
    try:
        with np.errstate(all="ignore"):
            pin(*args)
    except (AssertionError, ValueError, FloatingPointError, IndexError):
        return True
    return False


def test_real_oracle_passes_all_pins():
    for pin in DEFINITION_PINS:
        assert not _fails(pin, attention_ref), pin.__name__


@pytest.mark.parametrize("name", sorted(DEFINITION_MUTANTS))
def test_definition_mutant_is_caught(name):
    kw = DEFINITION_MUTANTS[name]
    mutant = lambda q, k, v, s, c: _definition(q, k, v, s, c, **kw)
    caught = [p.__name__ for p in DEFINITION_PINS if _fails(p, mutant)]
    assert caught, f"mutant {name} passed every pin"


@pytest.mark.parametrize("kind", ["no_acc_rescale", "no_l_rescale", "alpha_inverted", "stale_max"])
def test_recurrence_mutant_is_caught(kind):
    mutant = _tiled_mutant(kind)
    caught = _fails(pins.pin_worked_example_trace, mutant) or \
        _fails(lambda a, t: pins.pin_tiled_matches(a, t, quick=True), attention_ref, mutant)
    assert caught, f"recurrence mutant {kind} passed every pin"


def test_real_recurrence_passes():
    assert not _fails(pins.pin_worked_example_trace, tiled_ref)
