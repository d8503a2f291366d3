"""CPU check of the page lookup the fused extend kernel uses instead of a
division: with m = floor((2^32 - 1) / P), the multiply-high
q' = floor(t m / 2^32) is floor(t / P) or one less for every t < 2^32, so a
single correction (r = t - q' P; if r >= P: q' + 1, r - P) gives the exact
quotient and remainder.  Checked here for every page size the library
accepts up to 4096 (multiples of 16) and a few large ones, over token
indices up to 2^31 - 1: the ends of the range, the multiples of P and their
neighbours near the top, and a seeded random sample."""
import numpy as np


def _lookup(t: np.ndarray, P: int):
    m = np.uint64((2**32 - 1) // P)
    q = (t * m) >> np.uint64(32)
    r = t - q * np.uint64(P)
    fix = r >= P
    return q + fix, r - fix * np.uint64(P)


def test_multiply_high_page_lookup_is_exact():
    rng = np.random.default_rng(20261203)
    sizes = list(range(16, 4097, 16)) + [1600 * 7, 65536, 1 << 20, (1 << 24) + 16]
    top = np.uint64(2**31 - 1)
    for P in sizes:
        Pu = np.uint64(P)
        k = np.arange(1, 64, dtype=np.uint64)
        near = (top // Pu - k) * Pu
        t = np.concatenate([
            np.array([0, 1, P - 1, P, P + 1, 2**31 - 1, 2**31 - 2], dtype=np.uint64),
            near - 1, near, near + 1,
            rng.integers(0, 2**31, size=2000, dtype=np.int64).astype(np.uint64),
        ])
        q, r = _lookup(t, P)
        assert np.array_equal(q, t // Pu), P
        assert np.array_equal(r, t % Pu), P
