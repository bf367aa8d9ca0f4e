"""The synthetic workloads are seeded: their sizes are fixed, and the bench
line, the profiles and the parity tests all assume these values.  N and the
map size |map| (centre entries included, from the oracle) per layer that
builds a map; a change to a generator shows up here first."""
import functools

import numpy as np
import pytest

import oracle
import workloads


@functools.lru_cache(maxsize=None)
def _workload(index):
    return workloads.make_workload(index)

# (workload, layer) -> (N, |map|), K and channels as in the workload table
EXPECTED = {
    (0, 0): (5034, 53274),
    (1, 0): (150000, 374656),
    (2, 0): (79033, 455893),
    (3, 0): (79033, 455893),
    (3, 2): (34215, 228733),
    (3, 4): (12502, 79912),
    (3, 6): (4789, 33451),
    (4, 0): (640812, 3394074),
    (4, 1): (640812, 8883922),
}


@pytest.mark.parametrize("index,layer", sorted(EXPECTED))
def test_workload_sizes(index, layer):
    L = _workload(index).layers[layer]
    n, e = EXPECTED[(index, layer)]
    assert L.n == n
    assert oracle.build_map(L.coords, L.k).total_entries == e


def test_workload_layers_share_maps_where_chained():
    """Chained layers reuse the previous layer's coordinates (one map per
    U-Net level), and every layer's coordinates are unique rows."""
    for index in range(5):
        wl = _workload(index)
        for i, L in enumerate(wl.layers):
            assert np.unique(L.coords, axis=0).shape[0] == L.n
            if L.chain:
                assert np.array_equal(L.coords, wl.layers[i - 1].coords)
