"""Pins of the oracle's block selection: hand-worked cases, brute force over all subsets
on tiny arrays, and order properties on tie-heavy random arrays."""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import SELECT_THRESH_ABS, SELECT_THRESH_REL, SELECT_TOPK


@pytest.mark.parametrize("r,n,k", [(0.5, 16, 8), (0.5, 64, 32), (0.35, 256, 90), (0.5, 256, 128),
                                   (1.0, 7, 7), (1e-9, 9, 1), (0.25, 4, 1), (0.3, 10, 3),
                                   (0.31, 10, 4), (2.0, 5, 5)])
def test_keep_count(r, n, k):
    assert oracle.keep_count(r, n) == k


def test_topk_hand_cases():
    f = lambda x, r, ff=False: list(oracle.select_blocks(np.float32(x), SELECT_TOPK, r, ff))
    assert f([3, 1, 3, 2], 0.5) == [0, 2]
    assert f([3, 1, 3, 2], 0.75) == [0, 2, 3]
    assert f([1, 1, 1, 1], 0.5) == [0, 1]                  # ties: lower index wins
    assert f([float("nan"), 1, 2], 0.6) == [1, 2]          # NaN sorts last
    assert f([float("nan"), 1, 2], 1.0) == [0, 1, 2]
    assert f([0, 5, 4, 3], 0.5, True) == [0, 1]            # block 0 forced
    assert f([9, 5, 4, 3], 0.5, True) == [0, 1]
    assert f([0.0, -0.0, 1.0], 0.6) == [0, 2]              # -0 == +0: tie, index decides
    assert f([-0.0, 0.0, 1.0], 0.6) == [0, 2]
    assert f([5.0], 0.5) == [0]


def _brute_topk(x, k, force_first):
    """Best k-subset by exhaustive search: maximise the sorted score vector
    (NaN lowest), ties broken toward lower indices."""
    n = len(x)
    val = lambda m: -math.inf if math.isnan(x[m]) else x[m]
    best, best_key = None, None
    for sub in itertools.combinations(range(n), k):
        if force_first and 0 not in sub:
            continue
        others = [m for m in sub if not (force_first and m == 0)]
        vals = sorted(((val(m), -m, not math.isnan(x[m])) for m in others), reverse=True)
        key = [(v[2], v[0], v[1]) for v in vals]
        if best_key is None or key > best_key:
            best, best_key = sub, key
    return list(best)


def test_topk_brute_force_tie_heavy():
    rng = np.random.default_rng(4)
    levels = np.float32([0.0, 0.25, 0.5, 1.0, 2.0, 3.5, -1.0, np.nan])
    for trial in range(300):
        n = int(rng.integers(1, 9))
        x = rng.choice(levels, n)
        r = float(rng.choice([0.1, 0.3, 0.5, 0.7, 1.0]))
        ff = bool(rng.integers(0, 2))
        k = oracle.keep_count(r, n)
        got = list(oracle.select_blocks(x, SELECT_TOPK, r, ff))
        assert got == _brute_topk([float(v) for v in x], k, ff), (x, r, ff)


def test_topk_properties_random():
    rng = np.random.default_rng(8)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        x = rng.choice(np.float32([0.1, 0.2, 0.3, 0.4]), n) if trial % 2 else \
            rng.standard_normal(n).astype(np.float32)
        r = float(rng.uniform(0.01, 1.0))
        kept = oracle.select_blocks(x, SELECT_TOPK, r)
        assert len(kept) == oracle.keep_count(r, n)
        assert np.all(np.diff(kept) > 0)
        rest = np.setdiff1d(np.arange(n), kept)
        if len(rest):
            assert x[kept].min() >= x[rest].max()
            tie = x[kept].min()
            # among tied values the kept ones have the lowest indices
            tk = kept[x[kept] == tie]
            tr = rest[x[rest] == tie]
            if len(tr):
                assert tk.max() < tr.min()


def test_threshold_hand_cases():
    f = lambda x, mode, p, ff=False: list(oracle.select_blocks(np.float32(x), mode, p, ff))
    assert f([1, 2, 3, 4], SELECT_THRESH_REL, 1.0) == [2, 3]            # mean 2.5
    assert f([1, 2, 3, 4], SELECT_THRESH_REL, 0.75) == [1, 2, 3]        # T = 1.875
    assert f([1, 2, 3, 6], SELECT_THRESH_REL, 1.0) == [2, 3]            # T = 3.0, equality kept
    assert f([1, 2, 3, 4], SELECT_THRESH_REL, 0.8) == [2, 3]            # 0.8f*2.5 > 2
    assert f([1, 2, 3, 4], SELECT_THRESH_ABS, 3.0) == [2, 3]
    assert f([1, 2, 3, 4], SELECT_THRESH_ABS, 3.0, True) == [0, 2, 3]
    assert f([1, 1, 1], SELECT_THRESH_ABS, 2.0) == []                  # empty set allowed
    assert f([1, float("nan"), 3], SELECT_THRESH_REL, 1.0) == []       # NaN mean keeps nothing
    assert f([1, float("nan"), 3], SELECT_THRESH_REL, 1.0, True) == [0]
    assert f([1, float("nan"), 3], SELECT_THRESH_ABS, 2.0) == [2]      # NaN never kept


def test_threshold_mean_is_left_to_right_double():
    # 0.1f summed ten times left to right in double differs from the exact mean;
    # the threshold uses the sequential double sum.
    x = np.float32([0.1] * 10)
    total = 0.0
    for v in x:
        total += float(v)
    assert oracle.threshold_value(x, SELECT_THRESH_REL, 1.0) == total / 10
    kept = oracle.select_blocks(x, SELECT_THRESH_REL, 1.0)
    assert list(kept) == [m for m in range(10) if float(x[m]) >= total / 10]
