"""The backward oracle against its pins, and the pins against planted mistakes."""

import numpy as np
import pytest

import oracle_bwd_pins as pins
from oracle import (attention_bwd_cols_ref, attention_bwd_from_lse_ref, attention_bwd_ref,
                    attention_bwd_rows_ref, attention_ref, probabilities_ref)


@pytest.mark.parametrize("pin", pins.BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(attention_bwd_ref)


def _mutant(kind):
    """attention_bwd_ref with one plausible mistake planted."""
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        p, _, _, _ = probabilities_ref(q, k, scale, causal and kind != "mask_dropped")
        dv = (p @ do) if kind == "dv_untransposed" else (p.T @ do)
        dp = do @ v.T
        delta = dp.sum(axis=-1) if kind == "delta_rowsum_dp" else np.sum(p * dp, axis=-1)
        ds = p * dp if kind == "no_delta" else p * (dp - delta[:, None])
        dq = (1.0 if kind == "dq_unscaled" else scale) * ((ds.T if kind == "dq_transposed" else ds) @ k)
        dk = (1.0 if kind == "dk_unscaled" else scale) * ((ds if kind == "dk_untransposed" else ds.T) @ q)
        return dq, dk, dv, delta
    return bwd


MUTANTS = ["dv_untransposed", "delta_rowsum_dp", "no_delta", "dq_unscaled", "dk_unscaled",
           "dq_transposed", "dk_untransposed", "mask_dropped"]


def _fails(pin, impl):
    try:
        pin(impl)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("kind", MUTANTS)
def test_backward_mutant_is_caught(kind):
    caught = [p.__name__ for p in pins.BWD_PINS if _fails(p, _mutant(kind))]
    assert caught, f"backward mutant {kind} passed every pin"


@pytest.mark.parametrize("causal", [False, True])
def test_recompute_form_matches_definition(causal):
    """P from the saved LSE and D = O . dO give the same gradients."""
    rng = np.random.default_rng(7)
    n, d = 37, 16
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, lse = attention_ref(q, k, v, 0.25, causal)
    a = attention_bwd_ref(q, k, v, do, 0.25, causal)
    b = attention_bwd_from_lse_ref(q, k, v, o, lse, do, 0.25, causal)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_and_column_forms_match(causal):
    rng = np.random.default_rng(8)
    n, d = 45, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, 0.3, causal)
    rows = np.array([0, 1, 17, 44])
    np.testing.assert_allclose(attention_bwd_rows_ref(q, k, v, do, 0.3, causal, rows), dq[rows],
                               rtol=1e-12, atol=1e-13)
    cols = np.array([0, 5, 30, 44])
    ck, cv = attention_bwd_cols_ref(q, k, v, do, 0.3, causal, cols, block=16)
    np.testing.assert_allclose(ck, dk[cols], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cv, dv[cols], rtol=1e-12, atol=1e-13)
