"""Pins of the oracle's top-n selection: hand-derived golden cases, a library
sort, and exhaustive enumeration of subsets on tiny inputs."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import csa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "select_cases.json")


def _lexsort_top(scores, n):
    k = csa.keys(scores).astype(np.int64)
    order = np.lexsort((np.arange(k.size), -k))          # key desc, index asc
    return np.sort(order[:n]).astype(np.int32)


def test_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        s = np.array([float(v) for v in c["scores"]], np.float32)
        assert csa.select(s, c["n"]).tolist() == c["idx"], c


def test_matches_library_sort_with_heavy_ties(rng):
    pool = np.array([0.0, 1e-45, 3e-39, 1.0, 1.0, 2.5, np.inf, np.nan], np.float32)
    for C in (1, 2, 7, 64, 65, 300, 1031):
        s = pool[rng.integers(0, pool.size, C)]
        for n in sorted({0, 1, C // 3, C // 2, C - 1, C}):
            if n < 0:
                continue
            assert np.array_equal(csa.select(s, n), _lexsort_top(s, n))


def test_exhaustive_subsets_tiny(rng):
    for C in range(1, 8):
        for trial in range(6):
            s = rng.integers(0, 3, C).astype(np.float32)      # many ties
            k = csa.keys(s)
            for n in range(C + 1):
                good = []
                for sub in itertools.combinations(range(C), n):
                    S = set(sub)
                    ok = all(k[a] > k[b] or (k[a] == k[b] and a < b)
                             for a in S for b in range(C) if b not in S)
                    if ok:
                        good.append(list(sub))
                assert len(good) == 1                        # the result is unique
                assert csa.select(s, n).tolist() == good[0]


def test_rejects_out_of_range_n():
    with pytest.raises(ValueError):
        csa.select(np.ones(4, np.float32), 5)
    with pytest.raises(ValueError):
        csa.select(np.ones(4, np.float32), -1)


def test_nan_keys_are_canonical():
    s = np.array([np.nan, -np.nan, np.inf], np.float32)
    assert csa.keys(s).tolist() == [0x7FC00000, 0x7FC00000, 0x7F800000]
