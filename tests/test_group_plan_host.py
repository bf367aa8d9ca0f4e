"""The library's grouping planner (spconv_group_plan_counts, host code, no
device) against the oracle's adaptive grouping ("TorchSparse: regular
computation from irregular sparsity", sections "The spectrum: separate,
dense, grouped" and "How the groups are chosen"): the same groups in the same
order and the same padded rows on the page's worked columns, its special
cases and seeded random map sizes, and the argument checks."""
import math

import numpy as np
import pytest

import oracle
import submanifold_sparse_convolution_device_amd as sp

INF = float("inf")


def _same(counts, eps, S, centre=None):
    got, pad = sp.group_plan_counts(counts, eps, S, centre)
    ref = oracle.adaptive_groups(counts, eps, S, centre)
    assert got == ref, (counts, eps, S, centre)
    assert pad == oracle.padded_rows(counts, ref)
    return got


def test_slide_columns():
    counts = [3, 10, 2, 4, 3, 2, 4]
    for eps in (0.0, 0.125, 0.15, 0.19, 0.2, 0.25, 1.0):
        for S in (INF, 0.0, 4.0, 10.0, 11.0):
            _same(counts, eps, S)
    assert _same(counts, 0.15, INF) == [[1], [3, 6, 0, 4], [2, 5]]


@pytest.mark.parametrize("kv,centre", [(1, 0), (8, None), (27, 13), (125, 62), (343, 171)])
def test_random_map_sizes(kv, centre):
    rng = np.random.default_rng(kv)
    for trial in range(40):
        counts = rng.integers(0, 3000, size=kv)
        counts[rng.random(kv) < 0.2] = 0  # offsets without entries
        if trial % 5 == 0:
            counts = np.repeat(rng.integers(1, 50, size=(kv + 1) // 2), 2)[:kv]  # ties
        counts = [int(c) for c in counts]
        thresholds = [INF, 0.0, float(np.median(counts)), float(max(counts)), float(max(counts)) + 1]
        for eps in (0.0, 0.05, 0.2, 0.5, 1.0, float(rng.random())):
            for S in thresholds:
                _same(counts, eps, S, centre)


def test_large_counts_and_empty():
    counts = [2 ** 39, 2 ** 39 - 1, 7, 0, 2 ** 38]
    for eps in (0.0, 0.3, 0.5, 1.0):
        _same(counts, eps, INF)
    assert sp.group_plan_counts([0, 0, 0], 0.2, INF) == ([], 0)
    assert sp.group_plan_counts([0, 5, 0], 0.2, INF, centre=1) == ([[1]], 5)


def test_argument_checks():
    def status(*args, **kw):
        with pytest.raises(sp.SpconvError) as e:
            sp.spconv_group_plan_counts(*args, **kw)
        return e.value.name
    assert status([], 0.2, INF) == "SPCONV_ERR_INVALID_ARG"
    assert status([1] * 344, 0.2, INF) == "SPCONV_ERR_INVALID_ARG"
    assert status([1, 2, 3], 0.2, INF, centre=3) == "SPCONV_ERR_INVALID_ARG"
    assert status([1, 2, 3], 0.2, INF, centre=-2) == "SPCONV_ERR_INVALID_ARG"
    assert status([1, -2, 3], 0.2, INF) == "SPCONV_ERR_INVALID_ARG"
    assert status([1, 2 ** 40, 3], 0.2, INF) == "SPCONV_ERR_INVALID_ARG"
    for eps, S in ((-0.5, INF), (math.nan, INF), (0.2, -1.0), (0.2, math.nan)):
        assert status([1, 2, 3], eps, S) == "SPCONV_ERR_INVALID_ARG"
