"""The oracle against its pins (CPU only).

Every check here compares the oracle with something other than itself: the
pages' printed worked example, closed forms, invariants, scalar brute force,
and torch's SDPA in float64 (see ``oracle_pins.py``).
"""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
from oracle import attention_ref, attention_rows_ref, probabilities_ref, tiled_ref


def test_worked_example_value():
    pins.pin_worked_example_value(attention_ref)


def test_worked_example_trace():
    pins.pin_worked_example_trace(tiled_ref)


def test_worked_example_closed_form():
    pins.pin_worked_example_closed_form(attention_ref)
    pins.pin_worked_example_closed_form(lambda q, k, v, s, c: tiled_ref(q, k, v, s, c, 2, 3))


def test_uniform_scores():
    pins.pin_uniform_scores(attention_ref)


def test_constant_values():
    pins.pin_constant_values(attention_ref)


def test_single_key():
    pins.pin_single_key(attention_ref)


def test_row_stochastic():
    pins.pin_row_stochastic(probabilities_ref)


def test_shift_invariance():
    pins.pin_shift_invariance(attention_ref)


def test_permutation():
    pins.pin_permutation(attention_ref)


def test_large_scores():
    pins.pin_large_scores(attention_ref)


def test_brute_force():
    pins.pin_brute_force(attention_ref)


def test_library_sdpa():
    pins.pin_library_sdpa(attention_ref)


def test_tiled_matches_definition():
    pins.pin_tiled_matches(attention_ref, tiled_ref)


def test_tiled_on_all_pins():
    """The recurrence passes the same closed-form and invariant pins."""
    t = lambda q, k, v, s, c: tiled_ref(q, k, v, s, c, 4, 3)
    for pin in (pins.pin_uniform_scores, pins.pin_constant_values, pins.pin_single_key,
                pins.pin_shift_invariance, pins.pin_permutation, pins.pin_large_scores,
                pins.pin_brute_force):
        pin(t)


def test_rows_ref_matches_full():
    rng = np.random.default_rng(3)
    n, d = 70, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    rows = [0, 1, 17, 68, 69]
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.4, causal)
        orow, lrow = attention_rows_ref(q, k, v, 0.4, causal, rows)
        assert np.allclose(orow, o[rows], rtol=0, atol=1e-13)
        assert np.allclose(lrow, lse[rows], rtol=0, atol=1e-13)


def test_batched_leading_axes():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 3, 10, 4)) for _ in range(3))
    o, lse = attention_ref(q, k, v, 0.5, True)
    assert o.shape == (2, 3, 10, 4) and lse.shape == (2, 3, 10)
    o11, l11 = attention_ref(q[1, 2], k[1, 2], v[1, 2], 0.5, True)
    assert np.array_equal(o[1, 2], o11) and np.array_equal(lse[1, 2], l11)


def test_bf16_inputs_are_upcast_exactly():
    """bf16 values reach the oracle unchanged (bf16 -> fp64 is exact)."""
    import torch
    from workloads import make_qkv
    q, k, v = make_qkv(1, 2, 12, 8, torch.bfloat16, seed=9)
    qd = q.to(torch.float64).numpy()
    assert np.array_equal(qd.astype(np.float32).astype(np.float64), qd)
    o, _ = attention_ref(qd, k.to(torch.float64).numpy(), v.to(torch.float64).numpy(), 0.3, False)
    assert o.dtype == np.float64


def test_tile_sizes_must_be_positive():
    with pytest.raises(ValueError):
        tiled_ref(np.ones((2, 1)), np.ones((2, 1)), np.ones((2, 1)), 1.0, False, 0, 1)
