"""Host logic of the parity checks (tie classification), on the CPU."""
import numpy as np

import oracle as O
from parity import classify_row, rel_l2


def test_equal_rows_are_equal():
    s = np.array([0.4, 0.3, 0.2, 0.1])
    assert classify_row(s, 0.65, [0, 1])[0] == "equal"


def test_boundary_tie_accepts_neighbour_set():
    s = np.array([0.5, 0.25 + 4e-7, 0.25 - 4e-7])      # blocks 1 and 2 within 1e-6
    assert classify_row(s, 0.7, [0, 1])[0] == "equal"
    assert classify_row(s, 0.7, [0, 2])[0] == "tie"


def test_mass_tie_accepts_one_more_block():
    s = np.array([0.6, 0.3 + 2e-7, 0.1 - 2e-7])         # C_2 = 0.9 + 2e-7 vs p = 0.9
    p = float(np.float32(0.9))
    assert classify_row(s, p, [0, 1])[0] == "equal"
    assert classify_row(s, p, [0, 1, 2])[0] == "tie"


def test_clear_difference_fails():
    s = np.array([0.5, 0.3, 0.2])
    assert classify_row(s, 0.6, [0, 2])[0] == "fail"
    assert classify_row(s, 0.6, [0, 1, 2])[0] == "fail"


def test_rel_l2():
    assert rel_l2([1.0, 1.0], [1.0, 1.0]) == 0.0
    np.testing.assert_allclose(rel_l2([1.0, 0.0], [0.0, 1.0]), np.sqrt(2.0))
