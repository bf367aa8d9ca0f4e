"""Pins of the oracle's adaptive grouping ("TorchSparse: regular computation
from irregular sparsity", sections "The spectrum: separate, dense, grouped"
and "How the groups are chosen")."""
import numpy as np

import oracle
import workloads


def test_slide_example():
    """The slide's seven columns: the tallest keeps its own product, four of
    similar height are padded by two rows in all into one batch of four, the
    two shortest (equal) form a batch of two: three launches instead of seven,
    2 extra rows over the 28 real ones.  Heights consistent with that count:
    10, 4, 4, 3, 3, 2, 2 (in any kernel order)."""
    counts = [3, 10, 2, 4, 3, 2, 4]
    for eps in (0.125, 0.15, 0.19):
        g = oracle.adaptive_groups(counts, eps, float("inf"))
        assert g == [[1], [3, 6, 0, 4], [2, 5]]
        assert oracle.padded_rows(counts, g) - sum(counts) == 2 and sum(counts) == 28
    # at epsilon = 0.2 the first short column joins the four (ratio (5*4 - 16) / 20, exactly
    # 0.2: "at or below"); the second would bring it to 0.25 and starts a new group
    assert oracle.adaptive_groups(counts, 0.2, float("inf")) == [[1], [3, 6, 0, 4, 2], [5]]


def test_special_cases():
    """epsilon = 1, S unbounded: one dense batch; S = 0: separate products;
    epsilon = 0: equal map sizes only."""
    rng = np.random.default_rng(3)
    counts = [int(v) for v in rng.integers(1, 500, size=26)]
    assert oracle.adaptive_groups(counts, 1.0, float("inf")) == [sorted(range(26), key=lambda k: (-counts[k], k))]
    assert sorted(oracle.adaptive_groups(counts, 0.3, 0)) == [[k] for k in range(26)]
    for g in oracle.adaptive_groups(counts, 0.0, float("inf")):
        assert len(set(counts[k] for k in g)) == 1
    # S splits only the batches whose largest map reaches it
    big = oracle.adaptive_groups(counts, 0.5, float("inf"))
    split = oracle.adaptive_groups(counts, 0.5, 300)
    for g in big:
        if max(counts[k] for k in g) >= 300:
            assert all([k] in split for k in g)
        else:
            assert g in split


def test_symmetric_grouping_on_a_submanifold_map():
    """Map sizes of offsets d and -d are equal on a submanifold map, so
    epsilon = 0 pairs them: K = 3 gives 13 groups of two beside the centre
    (the paper's symmetric grouping), unless sizes coincide further."""
    c = workloads.random_grid(31, 20, 0.3, 1)
    m = oracle.build_map(c, 3)
    counts = [int(v) for v in m.counts]
    assert len(set(counts[k] for k in range(27) if k != 13)) == 13  # no coincidences here
    g = oracle.adaptive_groups(counts, 0.0, float("inf"), centre=13)
    assert g[0] == [13] and len(g) == 14
    for pair in g[1:]:
        assert len(pair) == 2 and pair[0] + pair[1] == 26


def test_empty_offsets_are_skipped():
    counts = [0, 5, 0, 5, 0]
    assert oracle.adaptive_groups(counts, 0.0, float("inf")) == [[1, 3]]
    assert oracle.adaptive_groups([0, 0, 7], 0.5, float("inf"), centre=2) == [[2]]
