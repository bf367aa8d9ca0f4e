"""Pins of the oracle's strided maps and their transposes (CPU).

The strided map follows "Sparse inputs and sparse convolution", section "The
map is the computation" (for each output q and offset d, look up s q + d),
with the outputs of the SparseConvNet blog's regular output definition
(section 2: an output is computed where the kernel covers at least one
active input).  Each pin below checks it against something the oracle does
not compute the same way: a brute-force enumeration of the definition, the
coordinate coarsening of the U-Net workload, the notes' dense growth at
stride 1, fp64 ``conv3d`` / ``conv_transpose3d`` on a dense grid, and the
adjoint identity.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads


def _lo(K):
    return -((K - 1) // 2)


def _offsets(K):
    lo = _lo(K)
    return [oracle.offset_of_any(k, K) for k in range(K ** 3)], lo


def _brute(coords, K, s):
    """Outputs and per-offset entry sets straight from the definition: every
    grid point q (in a box covering the inputs) whose window s q + D holds an
    input is an output; (j, q) is an entry of offset d when coords[j] =
    s q + d.  Outputs in lexicographic (b, z, y, x) order."""
    c = np.asarray(coords, dtype=np.int64)
    offs, lo = _offsets(K)
    present = {tuple(int(v) for v in r): i for i, r in enumerate(c)}
    hi = c[:, 1:].max() // s + 2
    outs = []
    for b in sorted(set(int(v) for v in c[:, 0])):
        for q in itertools.product(range(hi), repeat=3):
            if any((b, s * q[0] + d[0], s * q[1] + d[1], s * q[2] + d[2]) in present for d in offs):
                outs.append((b,) + q)
    lists = {k: set() for k in range(K ** 3)}
    for qi, q in enumerate(outs):
        for k, d in enumerate(offs):
            j = present.get((q[0], s * q[1] + d[0], s * q[2] + d[1], s * q[3] + d[2]))
            if j is not None:
                lists[k].add((j, qi))
    return np.array(outs, dtype=np.int64).reshape(-1, 4), lists


@pytest.mark.parametrize("K,s,seed", [(2, 2, 1), (3, 2, 2), (3, 1, 3), (2, 1, 4), (3, 3, 5), (4, 2, 6), (1, 2, 7)])
def test_strided_map_equals_the_definition(K, s, seed):
    c = workloads.permuted(workloads.random_grid(600 + seed, 9, 0.15, 2), seed)
    m = oracle.build_map_strided(c, K, s)
    outs, lists = _brute(c, K, s)
    assert m.N == c.shape[0] and m.N_out == outs.shape[0]
    assert np.array_equal(m.out_coords, outs)
    for k in range(K ** 3):
        a, b = m.lists[k]
        assert set(zip(a.tolist(), b.tolist())) == lists[k], f"offset {k}"
        assert np.all(np.diff(b) > 0)  # ordered by output row, one entry per output


def test_k2_stride2_is_the_coarsening():
    """K = 2, stride 2 with offsets {0, 1}^3: the outputs are exactly the
    U-Net workload's next level, unique((b, z//2, y//2, x//2)), and each
    input joins exactly one entry, at the offset of its remainder mod 2."""
    for seed in (11, 12):
        c = workloads.permuted(workloads.random_grid(seed, 16, 0.2, 2), seed)
        m = oracle.build_map_strided(c, 2, 2)
        assert np.array_equal(m.out_coords, workloads.coarsen(c))
        seen = np.zeros(m.N, np.int64)
        for k in range(8):
            a, b = m.lists[k]
            seen[a] += 1
            rem = c[a, 1:] % 2
            assert np.all(rem[:, 0] * 4 + rem[:, 1] * 2 + rem[:, 2] == k)
            assert np.array_equal(m.out_coords[b, 1:], c[a, 1:] // 2)
            assert np.array_equal(m.out_coords[b, 0], c[a, 0])
        assert np.all(seen == 1)
    lidar = workloads.make_workload(3).layers
    c0 = lidar[0].coords
    assert np.array_equal(oracle.build_map_strided(c0, 2, 2).out_coords, workloads.coarsen(c0))


def test_single_site():
    """One active site: 27 outputs at stride 1 with K = 3 (the notes' 1 -> 27
    in 3D); at stride 2 the outputs are the grid points whose window holds
    it, per axis those q with (p - d) / 2 integral for d in the kernel."""
    site = np.array([[0, 10, 11, 12]], np.int32)
    assert oracle.build_map_strided(site, 3, 1).N_out == 27
    assert oracle.build_map_strided(site, 2, 2).N_out == 1
    per_axis = [sum(1 for d in (-1, 0, 1) if (p - d) % 2 == 0) for p in (10, 11, 12)]
    assert oracle.build_map_strided(site, 3, 2).N_out == int(np.prod(per_axis)) == 2


def test_stride1_outputs_are_dense_growth():
    """At stride 1 the regular output definition grows the active set by one
    layer of the dense convolution ("Sparse inputs and sparse convolution",
    section "What a dense convolution does to empty space"), here on an
    unbounded grid (the inputs sit away from the origin)."""
    c = workloads.random_grid(21, 8, 0.1, 1).astype(np.int64)
    c[:, 1:] += 2
    m = oracle.build_map_strided(c, 3, 1)
    grown = oracle.dense_grow([tuple(r[1:]) for r in c], 1, None, K=3)
    assert set(tuple(int(v) for v in r[1:]) for r in m.out_coords) == grown
    assert m.N_out == len(grown)


def _dense(coords, feats, D):
    b = int(coords[:, 0].max()) + 1
    g = torch.zeros((b, feats.shape[1], D, D, D), dtype=torch.float64)
    c = torch.from_numpy(coords.astype(np.int64))
    g[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(feats)
    return g


def _conv_weight(W, K):
    # w[co, ci, kz, ky, kx] = W[k][ci][co], k = (kz K + ky) K + kx
    return torch.from_numpy(W).reshape(K, K, K, W.shape[1], W.shape[2]).permute(4, 3, 0, 1, 2).contiguous()


@pytest.mark.parametrize("K,s", [(2, 2), (3, 2), (3, 1), (4, 2)])
def test_strided_forward_equals_conv3d(K, s):
    """The strided forward equals fp64 conv3d with stride s and padding -lo
    on the zero-filled dense grid (output position o covers s o + lo .. s o
    + lo + K - 1), sampled at the output coordinates."""
    rng = np.random.default_rng(30 + K + s)
    c = workloads.permuted(workloads.random_grid(31 + K, 10, 0.2, 2), 3)
    m = oracle.build_map_strided(c, K, s)
    cin, cout = 3, 4
    f = rng.standard_normal((m.N, cin))
    W = rng.standard_normal((K ** 3, cin, cout))
    got = m.forward(f, W)
    D = 10 + K
    y = torch.nn.functional.conv3d(_dense(c, f, D), _conv_weight(W, K), stride=s, padding=-_lo(K))
    q = torch.from_numpy(m.out_coords.astype(np.int64))
    exp = y[q[:, 0], :, q[:, 1], q[:, 2], q[:, 3]].numpy()
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,s", [(2, 2), (3, 2), (3, 1)])
def test_transposed_forward_equals_conv_transpose3d(K, s):
    """The transposed map's forward (upsampling back onto the strided map's
    inputs) equals fp64 conv_transpose3d with the same stride and padding,
    sampled at the input coordinates; conv_transpose3d's weight [C_down,
    C_up, K, K, K] holds Wt[k][c_down][c_up]."""
    rng = np.random.default_rng(40 + K + s)
    c = workloads.permuted(workloads.random_grid(41 + K, 10, 0.2, 2), 4)
    m = oracle.build_map_strided(c, K, s)
    t = m.transpose()
    assert t.N == m.N_out and t.N_out == m.N
    cd, cu = 4, 3
    g = rng.standard_normal((t.N, cd))
    Wt = rng.standard_normal((K ** 3, cd, cu))
    got = t.forward(g, Wt)
    Dq = int(m.out_coords[:, 1:].max()) + 2
    w = torch.from_numpy(Wt).reshape(K, K, K, cd, cu).permute(3, 4, 0, 1, 2).contiguous()
    y = torch.nn.functional.conv_transpose3d(_dense(m.out_coords, g, Dq), w, stride=s, padding=-_lo(K))
    p = torch.from_numpy(c.astype(np.int64))
    exp = y[p[:, 0], :, p[:, 1], p[:, 2], p[:, 3]].numpy()
    assert np.allclose(got, exp, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,s", [(2, 2), (3, 2), (3, 1)])
def test_transpose_swaps_the_entries_and_is_the_adjoint(K, s):
    """Built from its own definition, the transposed map holds exactly the
    strided map's entries reversed, and with Wt[k] = W[k]^T its forward is the
    adjoint of the strided forward: <g, S f> = <T g, f>."""
    c = workloads.permuted(workloads.random_grid(51 + K, 9, 0.25, 2), 5)
    m = oracle.build_map_strided(c, K, s)
    t = m.transpose()
    assert np.array_equal(t.out_coords, c) and np.array_equal(t.coords, m.out_coords)
    for k in range(K ** 3):
        a, b = m.lists[k]
        ta, tb = t.lists[k]
        assert set(zip(ta.tolist(), tb.tolist())) == set(zip(b.tolist(), a.tolist()))
        assert np.all(np.diff(tb) > 0)
    rng = np.random.default_rng(52)
    f = rng.standard_normal((m.N, 5))
    g = rng.standard_normal((m.N_out, 6))
    W = rng.standard_normal((K ** 3, 5, 6))
    lhs = float(np.sum(g * m.forward(f, W)))
    rhs = float(np.sum(t.forward(g, np.ascontiguousarray(W.transpose(0, 2, 1))) * f))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_strided_map_errors():
    good = np.array([[0, 1, 2, 3], [0, 4, 5, 6]], np.int32)
    dup = np.array([[0, 1, 2, 3], [0, 1, 2, 3]], np.int32)
    far = np.array([[0, 1, 2, 70000]], np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.build_map_strided(dup, 2, 2)
    assert e.value.name == "DUPLICATE_COORD"
    with pytest.raises(oracle.OracleError) as e:
        oracle.build_map_strided(far, 2, 2)
    assert e.value.name == "COORD_RANGE"
    for K, s in ((0, 2), (8, 2), (3, 0), (3, 17)):
        with pytest.raises(oracle.OracleError) as e:
            oracle.build_map_strided(good, K, s)
        assert e.value.name == "INVALID_ARG"
    with pytest.raises(oracle.OracleError):
        oracle.build_map(good, 3).transpose()
