"""The CPU oracle against values it does not produce itself (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import tests.oracle_pins as P

finite32 = st.floats(min_value=-60.0, max_value=60.0, allow_nan=False, width=32)


def test_offsets_hand_example():
    P.pin_offsets_hand_example()


def test_mapping_hand_example():
    P.pin_mapping_hand_example()


@settings(max_examples=150, deadline=None)
@given(st.lists(finite32, min_size=1, max_size=16))
def test_logsoftmax_bruteforce(xs):
    P.pin_logsoftmax_bruteforce([xs])


def test_logsoftmax_closed_forms():
    P.pin_logsoftmax_closed_forms()


def test_logsoftmax_invariants():
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(n).astype(np.float32) * s
            for n, s in ((1, 1.0), (7, 3.0), (111, 1.5), (4096, 2.0), (32000, 1.0))]
    P.pin_logsoftmax_invariants(rows)


def test_worked_example():
    P.pin_worked_example()


@pytest.mark.parametrize("alphabet,vmax", [
    ((-np.inf, 0.0, 1.0), 7),
    ((-0.0, 0.0, 1.0), 6),
])
def test_ranking_exhaustive(alphabet, vmax):
    P.pin_ranking_exhaustive([float(a) for a in alphabet], vmax)


def test_ranking_special_cases():
    P.pin_ranking_special_cases()


def test_ranking_invariants():
    rng = np.random.default_rng(12)
    rows = [rng.integers(-4, 5, size=n).astype(np.float32) / 2 for n in (5, 40, 300, 5000)]
    rows += [rng.standard_normal(n).astype(np.float32) for n in (9, 1000)]
    P.pin_ranking_invariants(rows)


def test_batch_hand_example():
    P.pin_batch_hand_example()


def test_errors():
    P.pin_errors()


def test_levels_columns():
    P.pin_levels_columns()


def test_levels_bruteforce():
    rng = np.random.default_rng(13)
    rows = [rng.integers(-3, 4, size=n).astype(np.float32) / 2 for n in (1, 3, 20, 70, 130)]
    rows += [rng.standard_normal(n).astype(np.float32) for n in (2, 63, 64, 65, 200)]
    P.pin_levels_bruteforce(rows)


def test_levels_zero():
    P.pin_levels_zero()


def test_assembly_hand_examples():
    P.pin_assembly_hand_examples()


def test_assembly_worked_example():
    P.pin_assembly_worked_example()


def test_temperature():
    P.pin_temperature()


def test_top_k():
    P.pin_top_k()
