"""Pins the oracle to closed forms, invariants, brute force and an independent
library routine (torch conv3d in float64), chosen so that a dropped term, a
flipped sign, a wrong index or a transposed operand fails at least one test."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads


def _sets(m):
    return {k: set(zip(m.lists[k][0].tolist(), m.lists[k][1].tolist())) for k in range(m.K ** 3)}


# ---------------------------------------------------------------- map


def _cube(n, batches=(0,)):
    pts = [(b, z, y, x) for b in batches for z in range(n) for y in range(n) for x in range(n)]
    return np.array(pts, np.int32)


@pytest.mark.parametrize("K", [3, 5])
def test_cube_closed_form(K):
    """A fully active n^3 cube has count(d) = prod_i (n - |d_i|)."""
    n = 9
    m = oracle.build_map(_cube(n), K)
    for k in range(K ** 3):
        dz, dy, dx = oracle.offset_of(k, K)
        assert m.counts[k] == (n - abs(dz)) * (n - abs(dy)) * (n - abs(dx))


def test_cube_two_batches_never_mix():
    n = 6
    c = _cube(n, batches=(0, 1))
    m = oracle.build_map(c, 3)
    one = oracle.build_map(_cube(n), 3)
    assert np.array_equal(m.counts, 2 * one.counts)
    for k in range(27):
        j, q = m.lists[k]
        assert np.array_equal(c[j, 0], c[q, 0])


def test_isolated_points_only_centre():
    """Pairwise Chebyshev distance > r: only the centre entries exist."""
    pts = np.array([[0, 3 * i, 3 * j, 3 * l] for i in range(4) for j in range(4) for l in range(4)], np.int32)
    m = oracle.build_map(pts, 3)
    assert m.total_entries == pts.shape[0] == m.counts[13]
    m5 = oracle.build_map(pts, 5)  # distance 3 > r = 2 as well
    assert m5.total_entries == pts.shape[0]


@pytest.mark.parametrize("seed,extent,occ,batches,K", [
    (1, 6, 0.05, 1, 3), (2, 8, 0.2, 2, 3), (3, 7, 0.4, 1, 5), (4, 10, 0.1, 3, 3),
    (5, 6, 0.3, 1, 1), (6, 12, 0.05, 2, 5), (7, 9, 0.25, 1, 3),
])
def test_tree_lookup_matches_brute_force(seed, extent, occ, batches, K):
    c = workloads.random_grid(seed, extent, occ, batches)
    c = workloads.permuted(c, seed)  # row order must not matter
    m = oracle.build_map(c, K)
    assert _sets(m) == oracle.brute_map(c, K)


@pytest.mark.parametrize("seed,K", [(11, 3), (12, 5), (13, 3)])
def test_mirror_and_centre_invariants(seed, K):
    c = workloads.permuted(workloads.random_grid(seed, 10, 0.15, 2), seed)
    m = oracle.build_map(c, K)
    s = _sets(m)
    kv = K ** 3
    centre = kv // 2
    assert s[centre] == {(q, q) for q in range(c.shape[0])}
    for k in range(kv):
        # M_{-d} = {(q, j) : (j, q) in M_d}, and k(-d) = K^3 - 1 - k(d)
        assert s[kv - 1 - k] == {(q, j) for (j, q) in s[k]}
        assert m.counts[k] == m.counts[kv - 1 - k]
        for j, q in s[k]:
            d = c[j].astype(int) - c[q].astype(int)
            assert d[0] == 0 and oracle.offset_index(*d[1:], K) == k
    assert int((m.counts > 0).sum()) <= kv


def test_offset_index_convention():
    # dz slowest, dx fastest; centre = (K^3 - 1) / 2
    assert oracle.offset_index(-1, -1, -1, 3) == 0
    assert oracle.offset_index(0, 0, 0, 3) == 13
    assert oracle.offset_index(0, 0, 1, 3) == 14
    assert oracle.offset_index(0, 1, 0, 3) == 16
    assert oracle.offset_index(1, 0, 0, 3) == 22
    assert oracle.offset_index(0, 0, 0, 5) == 62
    for K in (1, 3, 5, 7):
        for k in range(K ** 3):
            assert oracle.offset_index(*oracle.offset_of(k, K), K) == k
            dz, dy, dx = oracle.offset_of(k, K)
            assert oracle.offset_index(-dz, -dy, -dx, K) == K ** 3 - 1 - k


# ---------------------------------------------------------------- forward


def _dense_conv3d_reference(coords, feats, w, K):
    """Zero-filled dense grid through torch conv3d (float64, cross-correlation,
    padding r), sampled at the active coordinates.  Weight layout:
    conv_w[co, ci, dz + r, dy + r, dx + r] = W[k(d)][ci][co]."""
    c = coords.astype(np.int64)
    r = (K - 1) // 2
    nb = int(c[:, 0].max()) + 1
    lo = c[:, 1:].min(axis=0)
    ext = c[:, 1:].max(axis=0) - lo + 1
    cin, cout = w.shape[1], w.shape[2]
    grid = torch.zeros((nb, cin, *ext.tolist()), dtype=torch.float64)
    idx = c[:, 1:] - lo
    grid[c[:, 0], :, idx[:, 0], idx[:, 1], idx[:, 2]] = torch.from_numpy(feats)
    cw = torch.from_numpy(w).reshape(K, K, K, cin, cout).permute(4, 3, 0, 1, 2).contiguous()
    y = torch.nn.functional.conv3d(grid, cw, padding=r)
    return y[c[:, 0], :, idx[:, 0], idx[:, 1], idx[:, 2]].numpy()


@pytest.mark.parametrize("seed,K,cin,cout,batches", [
    (21, 3, 5, 7, 1), (22, 3, 8, 3, 2), (23, 5, 4, 6, 1), (24, 1, 6, 5, 1), (25, 3, 16, 16, 1),
])
def test_forward_matches_dense_conv3d(seed, K, cin, cout, batches):
    c = workloads.permuted(workloads.random_grid(seed, 9, 0.2, batches), seed)
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((c.shape[0], cin))
    w = rng.standard_normal((K ** 3, cin, cout))
    m = oracle.build_map(c, K)
    got = m.forward(f, w)
    ref = _dense_conv3d_reference(c, f, w, K)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(got - ref)) <= 1e-12 * scale


def test_forward_rows_matches_full_forward():
    c = workloads.permuted(workloads.random_grid(31, 10, 0.2, 2), 31)
    rng = np.random.default_rng(31)
    f = rng.standard_normal((c.shape[0], 6))
    w = rng.standard_normal((27, 6, 4))
    m = oracle.build_map(c, 3)
    full = m.forward(f, w)
    rows = rng.choice(c.shape[0], 40, replace=False)
    assert np.allclose(m.forward_rows(f, w, rows), full[rows], rtol=0, atol=1e-12)
    t = oracle.build_table(c, 3)
    assert t.total_entries == 0
    assert np.allclose(t.forward_rows(f, w, rows), full[rows], rtol=0, atol=1e-12)
    assert np.array_equal(t.neighbours(rows), m.neighbours(rows))
    nbr = m.neighbours(rows)
    for i, q in enumerate(rows):
        for k in range(27):
            j, qq = m.lists[k]
            hit = j[qq == q]
            assert (hit.tolist() or [-1]) == [nbr[i, k]]


@pytest.mark.parametrize("threads", [0, 1, 2, 3, 7])
def test_forward_parallel_is_bit_identical(threads):
    """The row-parallel timing variant sums the same terms in the same order
    per output value as the serial forward (thread counts that do not divide
    the rows, more threads than needed, the runtime's default), and both agree
    with the dense conv3d reference."""
    c = workloads.permuted(workloads.random_grid(33, 11, 0.25, 2), 33)
    rng = np.random.default_rng(33)
    f = rng.standard_normal((c.shape[0], 12))
    w = rng.standard_normal((27, 12, 20))
    m = oracle.build_map(c, 3)
    serial = m.forward(f, w)
    par = m.forward_parallel(f, w, threads)
    assert np.array_equal(serial, par)
    tiny = np.array([[0, 1, 1, 1], [0, 1, 1, 2]], np.int32)
    mt = oracle.build_map(tiny, 3)
    ft, wt = rng.standard_normal((2, 4)), rng.standard_normal((27, 4, 4))
    assert np.array_equal(mt.forward(ft, wt), mt.forward_parallel(ft, wt, 5))
    ref = _dense_conv3d_reference(c, f, w, 3)
    assert np.max(np.abs(par - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_forward_routing_special_cases():
    c = workloads.random_grid(41, 8, 0.3, 1)
    n = c.shape[0]
    rng = np.random.default_rng(41)
    cin = 6
    f = rng.standard_normal((n, cin))
    m = oracle.build_map(c, 3)
    # (i) centre weight = identity, all others zero: output = input
    w = np.zeros((27, cin, cin))
    w[13] = np.eye(cin)
    assert np.array_equal(m.forward(f, w), f)
    # (ii) identity at one non-centre offset: a pure shift along the map
    for k in (0, 4, 17, 26):
        w = np.zeros((27, cin, cin))
        w[k] = np.eye(cin)
        got = m.forward(f, w)
        exp = np.zeros_like(f)
        j, q = m.lists[k]
        exp[q] = f[j]
        assert np.array_equal(got, exp)
    # (iii) all ones: f_out[q][c] = Cin * deg(q)
    ones = m.forward(np.ones((n, cin)), np.ones((27, cin, 3)))
    deg = np.zeros(n)
    for k in range(27):
        np.add.at(deg, m.lists[k][1], 1)
    assert np.array_equal(ones, np.repeat((cin * deg)[:, None], 3, axis=1))


def test_forward_k1_is_plain_gemm():
    c = workloads.random_grid(51, 7, 0.3, 1)
    rng = np.random.default_rng(51)
    f = rng.standard_normal((c.shape[0], 5))
    w = rng.standard_normal((1, 5, 9))
    m = oracle.build_map(c, 1)
    assert np.allclose(m.forward(f, w), f @ w[0], rtol=0, atol=1e-12)


def test_forward_linear_and_adjoint():
    """Linearity in f and W; adjoint <g, conv_W f> = <conv_W' g, f> with
    W'_d = (W_{-d})^T, which follows from the mirror map."""
    c = workloads.permuted(workloads.random_grid(61, 9, 0.25, 2), 61)
    n = c.shape[0]
    rng = np.random.default_rng(61)
    cin, cout = 5, 7
    m = oracle.build_map(c, 3)
    f1, f2 = rng.standard_normal((n, cin)), rng.standard_normal((n, cin))
    w1, w2 = rng.standard_normal((27, cin, cout)), rng.standard_normal((27, cin, cout))
    a, b = 0.7, -1.3
    lhs = m.forward(a * f1 + b * f2, w1)
    rhs = a * m.forward(f1, w1) + b * m.forward(f2, w1)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.abs(rhs).max()
    lhs = m.forward(f1, a * w1 + b * w2)
    rhs = a * m.forward(f1, w1) + b * m.forward(f1, w2)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.abs(rhs).max()
    g = rng.standard_normal((n, cout))
    wt = np.ascontiguousarray(np.transpose(w1[::-1], (0, 2, 1)))
    left = float(np.sum(g * m.forward(f1, w1)))
    right = float(np.sum(m.forward(g, wt) * f1))
    assert abs(left - right) <= 1e-10 * max(1.0, abs(left))


def test_synthetic_workload_statistics_small():
    """Workload shape sanity (statistics, not page values: parity unpinned for
    the generators themselves).  The sphere shell is deterministic."""
    wl = workloads.make_workload(0)
    layer = wl.layers[0]
    assert layer.n == 5034
    m = oracle.build_map(layer.coords, 3)
    assert m.counts[13] == layer.n
    assert m.total_entries == 53274


# ---------------------------------------------------------------- backward


def _dense_conv3d_grads(coords, feats, w, g, K):
    """Gradients of L = sum over active sites of <g, conv3d(zero-filled grid)>
    (torch float64 autograd) with respect to the active sites' input features
    and to the weights, the latter returned in the [K^3][Cin][Cout] layout."""
    c = coords.astype(np.int64)
    r = (K - 1) // 2
    nb = int(c[:, 0].max()) + 1
    lo = c[:, 1:].min(axis=0)
    ext = c[:, 1:].max(axis=0) - lo + 1
    cin, cout = w.shape[1], w.shape[2]
    idx = c[:, 1:] - lo
    grid = torch.zeros((nb, cin, *ext.tolist()), dtype=torch.float64)
    grid[c[:, 0], :, idx[:, 0], idx[:, 1], idx[:, 2]] = torch.from_numpy(feats)
    grid.requires_grad_(True)
    cw = torch.from_numpy(w).reshape(K, K, K, cin, cout).permute(4, 3, 0, 1, 2).contiguous().requires_grad_(True)
    y = torch.nn.functional.conv3d(grid, cw, padding=r)
    loss = (y[c[:, 0], :, idx[:, 0], idx[:, 1], idx[:, 2]] * torch.from_numpy(g)).sum()
    loss.backward()
    gin = grid.grad[c[:, 0], :, idx[:, 0], idx[:, 1], idx[:, 2]].numpy()
    gw = cw.grad.permute(2, 3, 4, 1, 0).reshape(K ** 3, cin, cout).numpy()
    return gin, gw


@pytest.mark.parametrize("seed,K,cin,cout,batches", [
    (61, 3, 5, 7, 1), (62, 3, 8, 3, 2), (63, 5, 4, 6, 1), (64, 1, 6, 5, 1), (65, 3, 16, 12, 1),
])
def test_backward_matches_dense_conv3d_autograd(seed, K, cin, cout, batches):
    """Both gradients equal torch's float64 conv3d backward on the zero-filled
    dense grid, read at the active sites (an independent library path)."""
    c = workloads.permuted(workloads.random_grid(seed, 9, 0.2, batches), seed)
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((c.shape[0], cin))
    w = rng.standard_normal((K ** 3, cin, cout))
    g = rng.standard_normal((c.shape[0], cout))
    m = oracle.build_map(c, K)
    gin_ref, gw_ref = _dense_conv3d_grads(c, f, w, g, K)
    gin = m.backward_data(g, w)
    gw = m.backward_weights(f, g)
    assert np.max(np.abs(gin - gin_ref)) <= 1e-12 * np.sqrt(np.mean(gin_ref ** 2))
    assert np.max(np.abs(gw - gw_ref)) <= 1e-12 * np.sqrt(np.mean(gw_ref ** 2))


def test_backward_adjoint_identities():
    """<g, conv_W f> = <backward_data(g, W), f> = <W, backward_weights(f, g)>:
    the forward is linear in f and in W, and the two gradients are its
    adjoints."""
    c = workloads.permuted(workloads.random_grid(66, 10, 0.25, 2), 66)
    rng = np.random.default_rng(66)
    f = rng.standard_normal((c.shape[0], 7))
    w = rng.standard_normal((27, 7, 5))
    g = rng.standard_normal((c.shape[0], 5))
    m = oracle.build_map(c, 3)
    lhs = float(np.sum(g * m.forward(f, w)))
    mid = float(np.sum(m.backward_data(g, w) * f))
    rhs = float(np.sum(w * m.backward_weights(f, g)))
    scale = float(np.sum(np.abs(g) * np.abs(m.forward(np.abs(f), np.abs(w)))))
    assert abs(lhs - mid) <= 1e-12 * scale and abs(lhs - rhs) <= 1e-12 * scale


def test_backward_data_is_forward_over_the_mirror():
    """The data gradient is the forward over the same map with the weights
    of the mirrored offset, transposed: W'_k = W_{K^3 - 1 - k}^T ("Sparse
    inputs and sparse convolution", section "A symmetry you can check on the
    slide": (P, Q, d) is an entry exactly when (Q, P, -d) is)."""
    for K in (3, 5):
        c = workloads.permuted(workloads.random_grid(67 + K, 9, 0.3, 1), 67)
        rng = np.random.default_rng(K)
        w = rng.standard_normal((K ** 3, 6, 9))
        g = rng.standard_normal((c.shape[0], 9))
        m = oracle.build_map(c, K)
        wm = np.ascontiguousarray(w[::-1].transpose(0, 2, 1))
        ref = m.forward(g, wm)
        assert np.max(np.abs(m.backward_data(g, w) - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2))


def test_backward_routing_special_cases():
    """Identity weights at one offset: the data gradient routes grad_out[q]
    back to the entry's input row (exactly); all-ones features and output
    gradients make the weight gradient of offset k its entry count."""
    c = workloads.random_grid(68, 8, 0.35, 1)
    n = c.shape[0]
    m = oracle.build_map(c, 3)
    rng = np.random.default_rng(68)
    g = rng.standard_normal((n, 4))
    for k in (13, 2, 20):
        w = np.zeros((27, 4, 4))
        w[k] = np.eye(4)
        exp = np.zeros((n, 4))
        j, q = m.lists[k]
        exp[j] = g[q]
        assert np.array_equal(m.backward_data(g, w), exp)
    gw = m.backward_weights(np.ones((n, 3)), np.ones((n, 2)))
    for k in range(27):
        assert np.all(gw[k] == m.counts[k])


@pytest.mark.parametrize("threads", [0, 1, 4, 30])
def test_backward_weights_parallel_is_bit_identical(threads):
    c = workloads.permuted(workloads.random_grid(69, 10, 0.3, 2), 69)
    rng = np.random.default_rng(69)
    f = rng.standard_normal((c.shape[0], 5))
    g = rng.standard_normal((c.shape[0], 6))
    m = oracle.build_map(c, 3)
    assert np.array_equal(m.backward_weights(f, g), m.backward_weights_parallel(f, g, threads))
