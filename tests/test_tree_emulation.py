"""The host emulation of the kernels' fixed norm tree (tests/parity_util.py),
which a GPU test compares with the library bit for bit, is itself a sum."""

import math

import numpy as np

from parity_util import fixed_tree_sum


def test_fixed_tree_emulation_is_a_sum():
    # Against math.fsum to the recursive-summation bound, on one block, one
    # level and two; sums of small integers are exact in any order.
    rng = np.random.default_rng(15)
    for n in (1, 7, 4096, 4097, 70_000, 4096 * 4096 + 9):
        x = rng.random(n)
        assert math.isclose(fixed_tree_sum(x), math.fsum(x.tolist()), rel_tol=1e-13), n
    assert fixed_tree_sum(np.zeros(0)) == 0.0
    assert fixed_tree_sum(np.ones(4097)) == 4097.0
    assert fixed_tree_sum(np.arange(70_000, dtype=np.float64)) == 70_000 * 69_999 / 2
