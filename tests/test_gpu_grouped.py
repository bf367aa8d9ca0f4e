"""GPU parity of the weight-stationary forward with adaptive grouping and of
the dataflow selector (through the C ABI).

Plans: the library's groups for (epsilon, S) equal ``oracle.adaptive_groups``
over the map's counts (same offsets, same order, same padded rows).
Forward: every output value within the forward's bound (|gpu - oracle| <=
tol x RMS + half an ulp, tol = 2e-2 for fp16 / bf16) against the oracle's
fp64 forward, for dense, separate, symmetric and mixed plans, submanifold,
strided and transposed maps, several tiles with ragged tails, and the
row-reordered map of the batched LiDAR frames.  Selector: its output is the
chosen dataflow's, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f16": 2e-2, "bf16": 2e-2}
HALF_ULP = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
INF = float("inf")


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


def _coords(c):
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV)


def _centre(kmap):
    return kmap.kernel_volume // 2 if kmap.kind == "submanifold" else None


def _check_out(got, ref, dtype):
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    diff = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    bound = TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref)
    assert np.all(diff <= bound), f"max |err| {float(diff.max()):.3e} vs RMS {rms:.3e}"


def _assert_plan(sp, kmap, eps, S):
    groups, pad = sp.group_plan(kmap, eps, S)
    ref = oracle.adaptive_groups(kmap.counts, eps, S, _centre(kmap))
    assert groups == ref, f"epsilon {eps}, S {S}"
    assert pad == oracle.padded_rows(kmap.counts, ref)
    return groups


PLANS = [(1.0, INF), (0.0, INF), (0.2, INF), (0.3, 2000.0), (0.5, 0.0)]


def test_group_plans_match_the_oracle(sp):
    """Submanifold maps (K = 1, 3, 5, rows permuted), a strided map and its
    transpose, over a grid of epsilon and S that includes the page's special
    cases (epsilon = 1, S = inf: one dense batch; S = 0: separate;
    epsilon = 0: equal sizes only) and thresholds at the maps' own sizes."""
    maps = []
    for K, seed in ((1, 1), (3, 2), (5, 3)):
        c = workloads.permuted(workloads.random_grid(800 + seed, 18, 0.2, 2), seed)
        maps.append(sp.build_map(_coords(c), K))
    c = workloads.permuted(workloads.random_grid(810, 20, 0.2, 2), 4)
    st = sp.build_map_strided(_coords(c), 3, 2)
    maps += [st, st.transpose()]
    for kmap in maps:
        counts = kmap.counts[kmap.counts > 0]
        thresholds = [INF, 0.0, float(np.median(counts)), float(counts.max()), float(counts.max()) + 1]
        for eps in (0.0, 0.05, 0.125, 0.2, 0.5, 1.0):
            for S in thresholds:
                _assert_plan(sp, kmap, eps, S)
    # the special cases, on the K = 3 submanifold map
    kmap = maps[1]
    c = _centre(kmap)
    nz = [k for k in range(27) if kmap.counts[k] > 0 and k != c]
    dense = _assert_plan(sp, kmap, 1.0, INF)
    assert dense[0] == [c] and sorted(dense[1]) == nz and len(dense) == 2
    sep = _assert_plan(sp, kmap, 0.3, 0.0)
    assert all(len(g) == 1 for g in sep) and len(sep) == len(nz) + 1
    sym = _assert_plan(sp, kmap, 0.0, INF)
    for g in sym[1:]:  # equal map sizes only: mirror pairs (or equal-sized pairs of pairs)
        assert len(set(int(kmap.counts[k]) for k in g)) == 1
        assert all(26 - k in g for k in g)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K,cin,cout", [(3, 32, 16), (3, 64, 64), (3, 96, 48), (3, 128, 128), (5, 64, 32),
                                        (3, 256, 256), (3, 512, 64), (1, 32, 32)])
def test_grouped_forward_random(sp, dtype, K, cin, cout):
    """Random grids (two batches, rows permuted: several 64-row tiles and a
    ragged last one) in every plan of PLANS, against the oracle's fp64
    forward; channel counts cover one to sixteen 32-channel chunks and
    weight slices of one to eight 16-column blocks."""
    seed = 830 + K + cin + cout
    c = workloads.permuted(workloads.random_grid(seed, 16, 0.25, 2), seed)
    ref = oracle.build_map(c, K)
    kmap = sp.build_map(_coords(c), K)
    assert kmap.n % 64 != 0
    f = workloads.features(ref.N, cin, dtype, seed + 1)
    w = workloads.weights(K, cin, cout, dtype, seed + 2)
    exp = ref.forward(f.double().numpy(), w.double().numpy())
    fd, wd = f.to(DEV), w.to(DEV)
    for eps, S in PLANS:
        got = sp.forward_grouped(fd, wd, kmap, eps, S).double().cpu().numpy()
        _check_out(got, exp, dtype)


def test_grouped_forward_is_repeatable_and_overwrites(sp):
    """Deterministic: the same bits on every call, whatever out held."""
    c = workloads.random_grid(840, 20, 0.2, 1)
    kmap = sp.build_map(_coords(c), 3)
    f = workloads.features(c.shape[0], 64, "bf16", 841).to(DEV)
    w = workloads.weights(3, 64, 64, "bf16", 842).to(DEV)
    out = torch.full((c.shape[0], 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    a = sp.forward_grouped(f, w, kmap, 0.2, INF, out=out).clone()
    b = sp.forward_grouped(f, w, kmap, 0.2, INF)
    assert torch.equal(a, b)


@pytest.mark.parametrize("K,s", [(2, 2), (3, 2), (3, 1)])
def test_grouped_strided_and_transposed(sp, K, s):
    """Maps without an identity offset: the strided forward (downsampling)
    and its transpose (upsampling) in the dense, separate and mixed plans."""
    seed = 850 + K * 3 + s
    c = workloads.permuted(workloads.random_grid(seed, 16, 0.25, 2), seed)
    ref = oracle.build_map_strided(c, K, s)
    kmap = sp.build_map_strided(_coords(c), K, s)
    t, tref = kmap.transpose(), ref.transpose()
    f = workloads.features(ref.N, 64, "bf16", seed + 1)
    w = workloads.weights(K, 64, 128, "bf16", seed + 2)
    g = workloads.features(ref.N_out, 128, "f16", seed + 3)
    wt = workloads.weights(K, 128, 32, "f16", seed + 4)
    down = ref.forward(f.double().numpy(), w.double().numpy())
    up = tref.forward(g.double().numpy(), wt.double().numpy())
    for eps, S in PLANS:
        _check_out(sp.forward_grouped(f.to(DEV), w.to(DEV), kmap, eps, S).double().cpu().numpy(), down, "bf16")
        _check_out(sp.forward_grouped(g.to(DEV), wt.to(DEV), t, eps, S).double().cpu().numpy(), up, "f16")


def test_grouped_unet_level3_c256(sp):
    """The U-Net workload's coarsest level (4,789 voxels, K = 3, C = 256,
    bf16) in every plan of PLANS, whole output against the oracle."""
    layer = [l for l in workloads.make_workload(3).layers if l.level == 3][0]
    ref = oracle.build_map(layer.coords, layer.k)
    kmap = sp.build_map(_coords(layer.coords), layer.k)
    f = workloads.features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
    w = workloads.weights(layer.k, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
    exp = ref.forward(f.double().numpy(), w.double().numpy())
    for eps, S in PLANS:
        got = sp.forward_grouped(f.to(DEV), w.to(DEV), kmap, eps, S).double().cpu().numpy()
        _check_out(got, exp, layer.dtype)


def test_grouped_batched_frames(sp):
    """8 batched LiDAR frames (640,812 voxels, K = 3, C = 128, bf16): a map
    whose rows the forward visits in its reordered sequence; the grouped
    forward in the symmetric and a mixed plan against the oracle's fp64
    forward on every output row."""
    layer = workloads.make_workload(4).layers[0]
    ref = oracle.build_map(layer.coords, layer.k)
    kmap = sp.build_map(_coords(layer.coords), layer.k)
    f = workloads.features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
    w = workloads.weights(layer.k, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
    exp = ref.forward_parallel(f.double().numpy(), w.double().numpy())
    for eps, S in ((0.0, INF), (0.3, 65536.0)):
        got = sp.forward_grouped(f.to(DEV), w.to(DEV), kmap, eps, S).double().cpu().numpy()
        _check_out(got, exp, layer.dtype)


def _distinct_plans(counts, centre, epsilons, thresholds):
    seen = []
    for S in thresholds:
        for eps in epsilons:
            g = oracle.adaptive_groups(counts, eps, S, centre)
            if g not in seen:
                seen.append(g)
    return len(seen)


def test_select_dataflow(sp):
    """The selector times the fused forward and every distinct plan of its
    grid, leaves the winner's output in out (the same bits as running the
    winner again) and reports a consistent choice."""
    c = workloads.random_grid(860, 24, 0.2, 1)
    kmap = sp.build_map(_coords(c), 3)
    f = workloads.features(c.shape[0], 64, "f16", 861).to(DEV)
    w = workloads.weights(3, 64, 64, "f16", 862).to(DEV)
    choice, out = sp.select_dataflow(f, w, kmap, reps=2)
    assert choice["dataflow"] in ("fused", "grouped")
    default_eps, default_S = [0.0, 0.1, 0.2, 0.3, 0.5, 1.0], [INF, 65536.0, 16384.0, 0.0]
    assert choice["candidates"] == 1 + _distinct_plans(kmap.counts, 13, default_eps, default_S)
    assert choice["ms"] > 0 and choice["fused_ms"] > 0 and choice["ms"] <= choice["fused_ms"]
    again = sp.forward_with(choice, f, w, kmap)
    assert torch.equal(out, again)
    if choice["dataflow"] == "grouped":
        assert choice["groups"] == len(oracle.adaptive_groups(kmap.counts, choice["epsilon"], choice["S"], 13))
    ref = oracle.build_map(c, 3).forward(f.double().cpu().numpy(), w.double().cpu().numpy())
    _check_out(out.double().cpu().numpy(), ref, "f16")
    # an explicit grid: one plan (S = 0: separate) besides the fused forward
    choice, out = sp.select_dataflow(f, w, kmap, epsilons=[0.0, 0.5], thresholds=[0.0], reps=1)
    assert choice["candidates"] == 2
    assert torch.equal(out, sp.forward_with(choice, f, w, kmap))
    # fp32: only the fused forward is a candidate
    f32 = f.float()
    choice, out = sp.select_dataflow(f32, w.float(), kmap, reps=1)
    assert choice["dataflow"] == "fused" and choice["candidates"] == 1


def test_grouped_empty_maps(sp):
    """A strided map without outputs: its grouped forward writes nothing and
    its transpose's writes zeros."""
    c = np.array([[0, 1, 3, 5], [0, 3, 3, 5], [1, 7, 1, 1]], np.int32)
    kmap = sp.build_map_strided(_coords(c), 1, 2)
    assert kmap.n == 0 and kmap.total_entries == 0
    f = torch.randn((3, 32), device=DEV).half()
    w = torch.randn((1, 32, 32), device=DEV).half()
    assert sp.forward_grouped(f, w, kmap, 0.2, INF).shape == (0, 32)
    assert sp.group_plan(kmap, 0.2, INF) == ([], 0)
    t = kmap.transpose()
    out = torch.full((3, 32), 7.0, device=DEV, dtype=torch.float16)
    sp.forward_grouped(torch.empty((0, 32), device=DEV, dtype=torch.float16), w, t, 0.2, INF, out=out)
    assert torch.count_nonzero(out).item() == 0


def test_grouped_errors(sp):
    c = workloads.random_grid(870, 10, 0.3, 1)
    kmap = sp.build_map(_coords(c), 3)
    n = c.shape[0]
    f = torch.zeros((n, 32), device=DEV, dtype=torch.float16)
    w = torch.zeros((27, 32, 32), device=DEV, dtype=torch.float16)
    for eps, S in ((-0.1, INF), (math.nan, INF), (0.2, -1.0), (0.2, math.nan)):
        with pytest.raises(sp.SpconvError) as e:
            sp.forward_grouped(f, w, kmap, eps, S)
        assert e.value.name == "SPCONV_ERR_INVALID_ARG"
        with pytest.raises(sp.SpconvError) as e:
            sp.group_plan(kmap, eps, S)
        assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    with pytest.raises(sp.SpconvError) as e:
        sp.forward_grouped(f.float(), w.float(), kmap, 0.2, INF)
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    f48 = torch.zeros((n, 48), device=DEV, dtype=torch.float16)
    with pytest.raises(sp.SpconvError) as e:
        sp.forward_grouped(f48, torch.zeros((27, 48, 32), device=DEV, dtype=torch.float16), kmap, 0.2, INF)
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    with pytest.raises(sp.SpconvError) as e:
        sp.forward_grouped(f, torch.zeros((27, 32, 24), device=DEV, dtype=torch.float16), kmap, 0.2, INF)
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    with pytest.raises(sp.SpconvError) as e:
        sp.select_dataflow(f, w, kmap, reps=0)
    assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    with pytest.raises(sp.SpconvError) as e:
        sp.select_dataflow(f, w, kmap, epsilons=[0.1, -1.0])
    assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    # NULL feature or output pointers with a map whose sides have rows
    out = torch.empty((n, 32), device=DEV, dtype=torch.float16)
    s = int(torch.cuda.current_stream().cuda_stream)
    for fn in (sp.spconv_forward, sp.spconv_forward_noalloc):
        with pytest.raises(sp.SpconvError) as e:
            fn(0, w.data_ptr(), kmap.handle, 32, 32, 1, out.data_ptr(), s)
        assert e.value.name == "SPCONV_ERR_INVALID_ARG"
        with pytest.raises(sp.SpconvError) as e:
            fn(f.data_ptr(), w.data_ptr(), kmap.handle, 32, 32, 1, 0, s)
        assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    with pytest.raises(sp.SpconvError) as e:
        sp.spconv_forward_grouped(0, w.data_ptr(), kmap.handle, 32, 32, 1, 0.2, INF, out.data_ptr(), s)
    assert e.value.name == "SPCONV_ERR_INVALID_ARG"
