"""The kernels divide small non-negative integers by a float reciprocal
instead of an integer division: floor((n + 0.5) * fl(1/d)) for n < 2^20 and
d <= 128 (tile indices from cell coordinates, a tile's cell and pixel rows,
task numbers). This pins that identity for every such pair in IEEE float32
arithmetic, the arithmetic the kernels use (an add that is exact below 2^23,
one rounded multiply, truncation toward zero)."""
import numpy as np


def test_float_reciprocal_division_is_exact():
    n = np.arange(1 << 20, dtype=np.int64)
    nf = n.astype(np.float32) + np.float32(0.5)
    assert np.all(nf - np.float32(0.5) == n.astype(np.float32))  # the add is exact
    for d in range(1, 129):
        inv = np.float32(1.0) / np.float32(d)
        q = (nf * inv).astype(np.int64)  # truncation, as the kernels' float -> int conversion
        bad = np.nonzero(q != n // d)[0]
        assert bad.size == 0, f"d={d}: first mismatch at n={int(bad[0])}"


def test_float_reciprocal_division_fails_without_the_half():
    # the + 0.5 is what makes it exact: without it some multiples of d
    # round just below the integer (a plausible slip this test would catch)
    n = np.arange(1 << 20, dtype=np.int64)
    misses = 0
    for d in range(1, 129):
        inv = np.float32(1.0) / np.float32(d)
        q = (n.astype(np.float32) * inv).astype(np.int64)
        misses += int(np.count_nonzero(q != n // d))
    assert misses > 0
