"""GPU parity of strided maps and their transposes (through the C ABI)
against the oracle.

Maps: the output coordinates bit-exact (lexicographic order), every offset's
list equal as a set and in increasing output row.  Forward: every output
value within the forward's bound (|gpu - oracle| <= tol x RMS + half an ulp,
tol = 2e-2 for fp16/bf16, 1e-5 for fp32).  Weight gradient: the bound of
test_gpu_backward.py (rounding chain of the summation).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_backward import _check_wgrad, _wgrad_rel

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


def _coords(c):
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV)


def _assert_map(kmap, ref):
    assert (kmap.n_in, kmap.n) == (ref.N, ref.N_out)
    assert np.array_equal(kmap.out_coords().cpu().numpy(), ref.out_coords)
    assert np.array_equal(kmap.counts, ref.counts)
    a, b = kmap.lists()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    off = kmap.offsets
    for k in range(ref.K ** 3):
        ga, gb = a[off[k]:off[k + 1]], b[off[k]:off[k + 1]]
        ra, rb = ref.lists[k]
        assert np.array_equal(gb, rb) and np.array_equal(ga, ra), f"offset {k}"


def _check_out(got, ref, dtype):
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    diff = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(diff <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref)), \
        f"max |err| {float(diff.max()):.3e} vs RMS {rms:.3e}"


CASES = [(2, 2), (3, 2), (3, 1), (1, 2), (4, 2), (5, 3), (2, 1)]


@pytest.mark.parametrize("K,s", CASES)
def test_strided_and_transposed_maps(sp, K, s):
    """Output coordinates and lists of the strided map and of its transpose,
    on two seeded random grids (rows in a random order, two batches)."""
    for seed in (700 + 10 * K + s, 701 + 10 * K + s):
        c = workloads.permuted(workloads.random_grid(seed, 13, 0.2, 2), seed)
        ref = oracle.build_map_strided(c, K, s)
        kmap = sp.build_map_strided(_coords(c), K, s)
        assert kmap.kind == "strided" and kmap.stride == s
        _assert_map(kmap, ref)
        t = kmap.transpose()
        assert t.kind == "transposed"
        _assert_map(t, ref.transpose())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K,s,cin,cout", [(2, 2, 32, 64), (3, 2, 64, 64), (3, 1, 16, 16), (2, 2, 128, 128),
                                          (3, 2, 32, 32), (2, 2, 256, 128), (3, 2, 48, 24)])
def test_strided_and_transposed_forward(sp, dtype, K, s, cin, cout):
    """Forward over the strided map (downsampling) and over its transpose
    (upsampling back) against the oracle's fp64 sums."""
    if dtype == "f32" and max(cin, cout) > 128:
        pytest.skip("fp32 kept to small channel counts")
    seed = 720 + K * 7 + s + cin
    c = workloads.permuted(workloads.random_grid(seed, 16, 0.25, 2), seed)
    ref = oracle.build_map_strided(c, K, s)
    kmap = sp.build_map_strided(_coords(c), K, s)
    f = workloads.features(ref.N, cin, dtype, seed + 1)
    w = workloads.weights(K, cin, cout, dtype, seed + 2)
    got = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    _check_out(got, ref.forward(f.double().numpy(), w.double().numpy()), dtype)
    t = kmap.transpose()
    tref = ref.transpose()
    g = workloads.features(ref.N_out, cout, dtype, seed + 3)
    wt = workloads.weights(K, cout, cin, dtype, seed + 4)
    got = sp.forward(g.to(DEV), wt.to(DEV), t).double().cpu().numpy()
    _check_out(got, tref.forward(g.double().numpy(), wt.double().numpy()), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_weight_gradient(sp, dtype):
    """Weight gradient over a strided map and its transpose (feature rows and
    gradient rows in different numbers)."""
    c = workloads.permuted(workloads.random_grid(740, 16, 0.25, 2), 740)
    ref = oracle.build_map_strided(c, 3, 2)
    kmap = sp.build_map_strided(_coords(c), 3, 2)
    for m, r in ((kmap, ref), (kmap.transpose(), ref.transpose())):
        f = workloads.features(r.N, 32, dtype, 741)
        g = workloads.features(r.N_out, 64, dtype, 742)
        gw = sp.backward_weights(f.to(DEV), g.to(DEV), m).double().cpu().numpy()
        fd, gd = f.double().numpy(), g.double().numpy()
        _check_wgrad(gw, r.backward_weights(fd, gd), r.backward_weights(np.abs(fd), np.abs(gd)),
                     _wgrad_rel(r.N_out, 3, 32, 64, dtype))


def test_unet_levels_are_the_strided_outputs(sp):
    """The U-Net workload's levels: a K = 2, stride 2 map of level l has the
    next level's coordinates as its outputs (the generator's coarsening), and
    the downsampling forward (C_l -> C_l+1, bf16) and the upsampling forward
    back match the oracle on every value."""
    layers = workloads.make_workload(3).layers
    levels = []
    for layer in layers:
        if not levels or layer.n != levels[-1].n:
            levels.append(layer)
    for lo_l, hi_l in zip(levels[:-1], levels[1:]):
        c = lo_l.coords
        ref = oracle.build_map_strided(c, 2, 2)
        kmap = sp.build_map_strided(_coords(c), 2, 2)
        assert np.array_equal(kmap.out_coords().cpu().numpy(), hi_l.coords)
        _assert_map(kmap, ref)
        f = workloads.features(lo_l.n, lo_l.cin, "bf16", 750)
        w = workloads.weights(2, lo_l.cin, hi_l.cin, "bf16", 751)
        got = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
        _check_out(got, ref.forward(f.double().numpy(), w.double().numpy()), "bf16")
        t = kmap.transpose()
        wt = workloads.weights(2, hi_l.cin, lo_l.cin, "bf16", 752)
        g = workloads.features(hi_l.n, hi_l.cin, "bf16", 753)
        got = sp.forward(g.to(DEV), wt.to(DEV), t).double().cpu().numpy()
        _check_out(got, ref.transpose().forward(g.double().numpy(), wt.double().numpy()), "bf16")


def test_batched_frames_downsampled(sp):
    """The 8 batched LiDAR frames (640,812 voxels): K = 2 / stride 2 and
    K = 3 / stride 2 maps compared in full with the oracle, and the bf16
    forward (64 -> 128 channels) on every value."""
    c = workloads.make_workload(4).layers[0].coords
    for K in (2, 3):
        ref = oracle.build_map_strided(c, K, 2)
        kmap = sp.build_map_strided(_coords(c), K, 2)
        _assert_map(kmap, ref)
        if K == 2:
            assert np.array_equal(ref.out_coords, workloads.coarsen(c))
    f = workloads.features(ref.N, 64, "bf16", 760)
    w = workloads.weights(3, 64, 128, "bf16", 761)
    got = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    _check_out(got, ref.forward_parallel(f.double().numpy(), w.double().numpy()), "bf16")


@pytest.mark.parametrize("K,s", [(3, 2), (2, 2), (5, 1)])
def test_widest_output_keys(sp, K, s):
    """Inputs at both ends of every coordinate range (b up to 2^15 - 1,
    z, y, x up to 2^16 - 1): the output keys need all their bits (every
    radix pass runs), and the map still equals the oracle's."""
    rng = np.random.default_rng(900 + K + s)
    lo = np.array([[0, 0, 0, 0]], np.int64) + rng.integers(0, 3, size=(12, 4))
    hi = np.array([[32767, 65535, 65535, 65535]], np.int64) - rng.integers(0, 3, size=(12, 4))
    c = np.unique(np.concatenate([lo, hi]), axis=0).astype(np.int32)
    c = workloads.permuted(c, 5)
    ref = oracle.build_map_strided(c, K, s)
    kmap = sp.build_map_strided(_coords(c), K, s)
    _assert_map(kmap, ref)
    _assert_map(kmap.transpose(), ref.transpose())


def test_no_outputs(sp):
    """A 1^3 kernel at stride 2 sees only inputs at even coordinates: with
    none, the map has no outputs; its forward writes nothing, its transpose's
    forward writes zeros and both weight gradients are zero."""
    c = np.array([[0, 1, 3, 5], [0, 3, 3, 5], [1, 7, 1, 1]], np.int32)
    kmap = sp.build_map_strided(_coords(c), 1, 2)
    assert (kmap.n_in, kmap.n, kmap.total_entries) == (3, 0, 0)
    f = torch.randn((3, 16), device=DEV).to(torch.float16)
    w = torch.randn((1, 16, 32), device=DEV).to(torch.float16)
    assert sp.forward(f, w, kmap).shape == (0, 32)
    t = kmap.transpose()
    assert (t.n_in, t.n, t.total_entries) == (0, 3, 0)
    out = torch.full((3, 16), 7.0, device=DEV, dtype=torch.float16)
    sp.forward(torch.empty((0, 32), device=DEV, dtype=torch.float16), torch.randn((1, 32, 16), device=DEV).half(),
               t, out=out)
    assert torch.count_nonzero(out).item() == 0
    gw = sp.backward_weights(f, torch.empty((0, 32), device=DEV, dtype=torch.float16), kmap)
    assert torch.count_nonzero(gw).item() == 0


def test_strided_errors(sp):
    dup = _coords(np.array([[0, 1, 2, 3], [0, 1, 2, 3]], np.int32))
    with pytest.raises(sp.SpconvError) as e:
        sp.build_map_strided(dup, 2, 2)
    assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
    far = _coords(np.array([[0, 1, 2, 70000]], np.int32))
    with pytest.raises(sp.SpconvError) as e:
        sp.build_map_strided(far, 2, 2)
    assert e.value.name == "SPCONV_ERR_COORD_RANGE"
    good = _coords(np.array([[0, 1, 2, 3], [0, 4, 5, 6]], np.int32))
    for K, s in ((0, 2), (6, 2), (3, 0), (3, 17)):
        with pytest.raises(sp.SpconvError) as e:
            sp.build_map_strided(good, K, s)
        assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    sub = sp.build_map(good, 3)
    with pytest.raises(sp.SpconvError) as e:
        sub.transpose()
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    kmap = sp.build_map_strided(good, 3, 2)
    g = torch.zeros((kmap.n, 16), device=DEV, dtype=torch.float16)
    w = torch.zeros((27, 16, 16), device=DEV, dtype=torch.float16)
    with pytest.raises(sp.SpconvError) as e:
        sp.backward_data(g, w, kmap)
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
