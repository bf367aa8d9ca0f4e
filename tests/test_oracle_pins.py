"""Pins the oracle to what the pages print: worked examples, quiz answers and
cost tables (fixtures under tests/golden/, each with its citation).

Page conventions: the 2D examples use (row, column) and W(dx, dy) with dx the
row offset and dy the column offset, input P = output Q + (dx, dy).  A 2D
example is embedded in 3D as b = 0, z = 0, y = row, x = column, so the page's
W(dx, dy) is this library's offset (dz, dy, dx) = (0, page dx, page dy).
"""
import json
import os

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _embed(points):
    return np.array([[0, 0, r, c] for r, c in points], dtype=np.int32)


def _page_weight(label):
    # "W(dx,dy)" -> (dx, dy)
    a, b = label[2:-1].split(",")
    return int(a), int(b)


def _as_sets(m):
    return {k: set(zip(m.lists[k][0].tolist(), m.lists[k][1].tolist())) for k in range(m.K ** 3)}


def test_worked_5x5_map_exact():
    g = _load("worked_5x5_map.json")
    names = sorted(g["points"], key=lambda s: int(s[1:]))
    coords = _embed([g["points"][n] for n in names])
    m = oracle.build_map(coords, 3)
    got = _as_sets(m)
    expected = {k: set() for k in range(27)}
    for label, entries in g["groups"].items():
        dx, dy = _page_weight(label)
        k = oracle.offset_index(0, dx, dy, 3)
        for p, q in entries:
            expected[k].add((int(p[1:]), int(q[1:])))
    assert got == expected
    assert m.total_entries == g["total_entries"]
    nonempty = [k for k in range(27) if m.counts[k] > 0]
    assert len(nonempty) == g["matmuls"]
    # offsets in the page's listing order (lexicographic in (dx, dy)) have 2, 1, 5, 1, 2 rows
    assert [int(m.counts[k]) for k in nonempty] == g["rows_per_matmul"]
    # in-plane offsets: 9 possible, 4 empty
    plane = [oracle.offset_index(0, a, b, 3) for a in (-1, 0, 1) for b in (-1, 0, 1)]
    assert sum(1 for k in plane if m.counts[k] == 0) == g["empty_offsets"]


def test_worked_5x5_lists_ordered_by_output():
    g = _load("worked_5x5_map.json")
    names = sorted(g["points"], key=lambda s: int(s[1:]))
    m = oracle.build_map(_embed([g["points"][n] for n in names]), 3)
    for k in range(27):
        outs = m.lists[k][1]
        assert np.all(np.diff(outs) > 0)


def test_quiz_sign_convention():
    q = _load("dilation_and_quiz.json")["quiz_sign"]
    # input at (3, 2), weight W(1, 0): the output is at input - offset
    p = q["input"]
    dx, dy = q["weight"]
    expect_q = q["output"]
    coords = _embed([p, expect_q])
    m = oracle.build_map(coords, 3)
    k = oracle.offset_index(0, dx, dy, 3)
    assert set(zip(m.lists[k][0].tolist(), m.lists[k][1].tolist())) == {(0, 1)}
    # the opposite sign convention would put the entry under W(-1, 0)
    k_wrong = oracle.offset_index(0, -dx, -dy, 3)
    assert set(zip(m.lists[k_wrong][0].tolist(), m.lists[k_wrong][1].tolist())) == {(1, 0)}


def test_p0_nine_entries_become_two():
    g = _load("grid_4x5.json")
    coords = _embed(g["active"])
    m = oracle.build_map(coords, 3)
    p0 = g["active"].index(g["p0"])
    as_input = [(k, q) for k in range(27) for j, q in zip(*[a.tolist() for a in m.lists[k]]) if j == p0]
    assert len(as_input) == g["p0_entries_submanifold"]
    partner = g["active"].index(g["p0_submanifold_partner"]["output"])
    dx, dy = _page_weight(g["p0_submanifold_partner"]["weight"])
    assert (oracle.offset_index(0, dx, dy, 3), partner) in as_input
    assert (13, p0) in as_input
    # conventionally P0 lands in nine output windows
    assert oracle.conventional_entries([g["p0"]], tuple(g["shape"])) == g["p0_entries_conventional"]


def test_4x5_cost_table():
    g = _load("grid_4x5.json")
    shape = tuple(g["shape"])
    m = oracle.build_map(_embed(g["active"]), 3)
    c = g["channels"]
    assert c * c == g["macs_per_entry"]
    sub = g["cost_table"]["submanifold"]
    assert m.total_entries == sub["entries"]
    assert oracle.mac_count(m.total_entries, c, c) == sub["macs"]
    conv = g["cost_table"]["conventional_zero_skip"]
    assert oracle.conventional_entries(g["active"], shape) == conv["entries"]
    assert oracle.mac_count(conv["entries"], c, c) == conv["macs"]
    dense = g["cost_table"]["fully_dense"]
    assert shape[0] * shape[1] * 9 == dense["entries"]
    assert oracle.mac_count(dense["entries"], c, c) == dense["macs"]
    # per-point clipped windows 9, 9, 6, 6
    assert [oracle.conventional_entries([a], shape) for a in g["active"]] == g["windows_per_point_clipped"]
    # the submanifold map: 4 centre entries plus each neighbour pair in both directions
    pairs = {tuple(sorted((tuple(a), tuple(b)))) for a, b in g["neighbour_pairs"]}
    act = [tuple(a) for a in g["active"]]
    got_pairs = set()
    for k in range(27):
        if k == 13:
            continue
        for j, q in zip(*[a.tolist() for a in m.lists[k]]):
            got_pairs.add(tuple(sorted((act[j], act[q]))))
    assert got_pairs == pairs
    assert m.total_entries == len(act) + 2 * len(pairs)
    # derived per-offset counts: W(-1,-1) = W(1,1) = 2, W(-1,1) = W(1,-1) = 1
    idx = lambda a, b: oracle.offset_index(0, a, b, 3)
    assert (m.counts[idx(-1, -1)], m.counts[idx(1, 1)], m.counts[idx(-1, 1)], m.counts[idx(1, -1)]) == (2, 2, 1, 1)
    # submanifold outputs = inputs (quiz: four outputs)
    assert len(set(m.lists[13][1].tolist())) == g["submanifold_outputs"]


def test_dense_growth_4x5():
    g = _load("grid_4x5.json")
    shape = tuple(g["shape"])
    one = oracle.dense_grow(g["active"], 1, shape)
    assert len(one) == g["dense_after_one_layer"]
    empty = {(r, c) for r in range(shape[0]) for c in range(shape[1])} - one
    assert empty == {tuple(e) for e in g["empty_after_one_layer"]}
    assert len(oracle.dense_grow(g["active"], 2, shape)) == g["dense_after_two_layers"]


def test_dilation_counts_single_site():
    d = _load("dilation_and_quiz.json")
    assert [len(oracle.dense_grow([(0, 0)], L)) for L in range(3)] == d["single_site_2d"]
    assert [len(oracle.dense_grow([(0, 0, 0)], L)) for L in range(3)] == d["single_site_3d"]
    assert len(oracle.dense_grow([(5, 5, 5)], 2)) == d["quiz_two_dense_3x3x3_layers"]
    for dim in (1, 2, 3):
        for L in range(4):
            assert len(oracle.dense_grow([(0,) * dim], L)) == (2 * L + 1) ** dim


def test_submanifold_output_count_is_constant():
    """Outputs are the inputs after any number of layers, while the dense
    definition grows (4 -> 17 -> 20 on the slide grid)."""
    g = _load("grid_4x5.json")
    coords = _embed(g["active"])
    for _ in range(100):
        m = oracle.build_map(coords, 3)
        outs = set(np.concatenate([m.lists[k][1] for k in range(27)]).tolist())
        assert outs == set(range(len(g["active"])))
        # the next layer's coordinate set is this layer's output set, i.e. unchanged
        coords = coords[sorted(outs)]
    assert coords.shape[0] == g["submanifold_outputs"]


def test_weight_stationary_matmul_count():
    d = _load("dilation_and_quiz.json")
    g = _load("worked_5x5_map.json")
    names = sorted(g["points"], key=lambda s: int(s[1:]))
    m = oracle.build_map(_embed([g["points"][n] for n in names]), 3)
    assert int((m.counts > 0).sum()) == d["quiz_weight_stationary_matmuls"]


def test_error_statuses():
    ok = np.array([[0, 1, 2, 3], [0, 1, 2, 4]], np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.build_map(np.array([[0, 1, 2, 3], [0, 1, 2, 3]], np.int32), 3)
    assert e.value.name == "DUPLICATE_COORD"
    for bad in ([0, -1, 0, 0], [0, 0, 65536, 0], [0, 0, 0, 70000], [32768, 0, 0, 0], [-1, 0, 0, 0]):
        with pytest.raises(oracle.OracleError) as e:
            oracle.build_map(np.array([[0, 0, 0, 0], bad], np.int32), 3)
        assert e.value.name == "COORD_RANGE"
    for K in (0, 2, 4, -3):
        with pytest.raises(oracle.OracleError) as e:
            oracle.build_map(ok, K)
        assert e.value.name == "INVALID_ARG"
    # extreme in-range coordinates are accepted; neighbours beyond the range are misses, never wraps
    edge = np.array([[32767, 65535, 65535, 65535], [32767, 0, 0, 0], [0, 65535, 65535, 65535]], np.int32)
    m = oracle.build_map(edge, 3)
    assert m.total_entries == 3
