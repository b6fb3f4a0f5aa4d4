"""The oracle's plain-C twin (``oracle/tiled_ref.c``) against the pins (CPU).

The C file restates the recurrence of ``oracle/tiled.py`` in fp64 C; it is
timed by bench.py as a second CPU baseline.  Like the Python oracle it is
pinned to facts outside itself (``oracle_pins.py``): the pages' worked
example, closed forms, invariants, scalar brute force, torch's SDPA in
float64 and the plain definition for many tile sizes.  Planted mistakes in
compiled copies of the C source must each fail at least one pin.
"""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention_ref
from oracle import native


def _attn(Br, Bc):
    return lambda q, k, v, s, c: native.tiled_ref_c(q, k, v, s, c, Br, Bc)


TILES = [(1, 1), (2, 3), (7, 16), (64, 64)]


@pytest.mark.parametrize("Br,Bc", TILES)
def test_worked_example(Br, Bc):
    pins.pin_worked_example_value(_attn(Br, Bc))
    pins.pin_worked_example_closed_form(_attn(Br, Bc))


@pytest.mark.parametrize("Br,Bc", TILES)
def test_closed_forms(Br, Bc):
    pins.pin_uniform_scores(_attn(Br, Bc))
    pins.pin_constant_values(_attn(Br, Bc))
    pins.pin_single_key(_attn(Br, Bc))


@pytest.mark.parametrize("Br,Bc", TILES)
def test_invariants(Br, Bc):
    pins.pin_shift_invariance(_attn(Br, Bc))
    pins.pin_permutation(_attn(Br, Bc))
    pins.pin_large_scores(_attn(Br, Bc))


@pytest.mark.parametrize("Br,Bc", [(1, 1), (2, 3), (16, 5)])
def test_brute_force(Br, Bc):
    pins.pin_brute_force(_attn(Br, Bc))


def test_library_sdpa():
    pins.pin_library_sdpa(_attn(8, 5))


def test_tile_sizes_reach_the_definition():
    pins.pin_tiled_matches(attention_ref, lambda q, k, v, s, c, Br, Bc, trace=None: native.tiled_ref_c(
        q, k, v, s, c, Br, Bc))


def test_row_ranges():
    """Any range of query rows, with tiles starting at its first row, gives
    those rows of the whole-head result."""
    rng = np.random.default_rng(31)
    n, d = 203, 12
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = native.tiled_ref_c(q, k, v, 0.3, causal, 16, 32)
        for r0, r1 in ((0, 1), (5, 77), (150, 203), (202, 203), (40, 40)):
            o2, l2 = native.tiled_rows_c(q, k, v, 0.3, causal, 7, 9, r0, r1)
            assert np.allclose(o2, o[r0:r1], rtol=0, atol=1e-13)
            assert np.allclose(l2, lse[r0:r1], rtol=0, atol=1e-13)


def test_bad_arguments():
    q = np.zeros((4, 2))
    with pytest.raises(ValueError):
        native.tiled_rows_c(q, q, q, 1.0, False, 0, 2, 0, 4)
    with pytest.raises(ValueError):
        native.tiled_rows_c(q, q, q, 1.0, False, 2, 2, 3, 5)


MUTANTS = {
    "acc not rescaled": [("for (long e = 0; e < d; ++e) acc[r * d + e] *= alpha;", "")],
    "l not rescaled": [("l[r] *= alpha;", "")],
    "inverted alpha": [("exp(m[r] - ref)", "exp(ref - m[r])")],
    "stale max": [("m[r] = m_new;", "")],
    "strict causal mask": [("if (!causal || j <= i) {", "if (!causal || j < i) {")],
    "dropped scale": [("x *= scale;", "")],
    "transposed scores": [("q[i * d + e] * k[j * d + e]", "q[j * d + e] * k[i * d + e]")],
    "wrong value row": [("p * v[j * d + e]", "p * v[i * d + e]")],
    "LSE without the max": [("lse[i] = m[r] + log(l[r]);", "lse[i] = log(l[r]);")],
    "LSE in base 2": [("lse[i] = m[r] + log(l[r]);", "lse[i] = m[r] + log2(l[r]);")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(name):
    lib = native.mutant_library(MUTANTS[name])

    def attn(q, k, v, s, c):
        return native.tiled_ref_c(q, k, v, s, c, 2, 3, lib=lib)

    checks = [pins.pin_worked_example_value, pins.pin_worked_example_closed_form, pins.pin_uniform_scores,
              pins.pin_constant_values, pins.pin_single_key, pins.pin_shift_invariance, pins.pin_brute_force]
    failed = []
    for pin in checks:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"
