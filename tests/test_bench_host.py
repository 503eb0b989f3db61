"""Host-side helpers of bench.py against the pinned oracle (CPU)."""
import math

import numpy as np

import bench
import oracle


def test_reuse_overlap_matches_the_oracle():
    """The overlap the benchmark reports equals oracle.overlap_fraction(own,
    reused) row by row: random ascending -1-padded selections, full rows,
    disjoint and empty ones."""
    r = np.random.default_rng(7)
    cases = [(np.array([3, 7, 9, -1]), np.array([1, 3, 9, 11])),
             (np.full(4, -1), np.array([1, 2, 3, 4])),
             (np.array([1, 2, 3, 4]), np.full(4, -1)),
             (np.arange(6), np.arange(6))]
    for _ in range(300):
        k = int(r.integers(1, 16))
        L = int(r.integers(k, 64))
        sel = []
        for _ in range(2):
            n = int(r.integers(0, k + 1))
            x = np.full(k, -1, dtype=np.int32)
            x[:n] = np.sort(r.choice(L, size=n, replace=False))
            sel.append(x)
        cases.append(tuple(sel))
    for own, reused in cases:
        want = oracle.overlap_fraction(own, reused)
        got = bench.reuse_overlap(own[None, :], reused[None, :])
        assert (math.isnan(want) and math.isnan(got)) or got == want, (own, reused, got, want)
