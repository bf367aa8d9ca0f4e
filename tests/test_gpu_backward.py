"""GPU parity of the backward through the C ABI against the oracle.

Data gradient: in the feature dtype, held to the forward's bound
(|gpu - oracle| <= tol x RMS(oracle) + half an ulp of the oracle's value,
tol = 2e-2 for fp16/bf16 and 1e-5 for fp32).

Weight gradient: fp32 output of sums of exactly representable products of
the stored inputs, accumulated in fp32 in three levels: 32 products inside
an MFMA (or 32 fused multiply-adds), at most 512 such steps per chunk of
16384 entries, and at most ceil(N / 16384) chunks.  The rounding error of
such a sum is at most (31 + 512 + chunks) unit roundoffs times the sum of the
terms' magnitudes, so each value is checked against
2^-14 x sum_e |f[j_e][ci]| |g[q_e][co]| (2^-14 = 1024 x 2^-24), that sum
coming from the oracle run on |f| and |g|; fp32 inputs add one rounding per
product, within the same bound.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
WGRAD_REL = 2.0 ** -14


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


def _map(sp, c, K):
    return sp.build_map(torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV), K)


def _check_dgrad(got, ref, dtype):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    diff = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(diff <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref)), \
        f"max |err| {float(diff.max()):.3e} vs RMS {rms:.3e}"


def _check_wgrad(got, ref, bound_terms):
    diff = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    bound = WGRAD_REL * bound_terms
    worst = int(np.argmax(diff - bound))
    assert np.all(diff <= bound), (f"|err| {diff.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} "
                                   f"(ref {ref.flat[worst]:.3e})")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K,cin,cout", [(3, 16, 16), (3, 32, 32), (3, 32, 16), (1, 32, 32), (3, 64, 64),
                                        (3, 128, 128), (3, 48, 24), (5, 32, 64), (3, 256, 256), (3, 8, 40)])
def test_backward_random_grids(sp, dtype, K, cin, cout):
    if dtype == "f32" and (cin > 128 or cout > 128):
        pytest.skip("fp32 kept to small channel counts")
    seed = 500 + K * 7 + cin + cout
    c = workloads.permuted(workloads.random_grid(seed, 14, 0.2, 2), seed)
    n = c.shape[0]
    ref = oracle.build_map(c, K)
    kmap = _map(sp, c, K)
    f = workloads.features(n, cin, dtype, seed + 1)
    g = workloads.features(n, cout, dtype, seed + 2)
    w = workloads.weights(K, cin, cout, dtype, seed + 3)
    gin = sp.backward_data(g.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    _check_dgrad(gin, ref.backward_data(g.double().numpy(), w.double().numpy()), dtype)
    gw = sp.backward_weights(f.to(DEV), g.to(DEV), kmap).double().cpu().numpy()
    fd, gd = f.double().numpy(), g.double().numpy()
    _check_wgrad(gw, ref.backward_weights(fd, gd), ref.backward_weights(np.abs(fd), np.abs(gd)))


def test_backward_routing_and_counts_exact(sp):
    """Identity weights at one offset send grad_out[q] back to the entry's
    input row exactly; all-ones inputs make every weight gradient of offset
    k equal its entry count."""
    c = workloads.permuted(workloads.random_grid(520, 12, 0.3, 1), 520)
    n = c.shape[0]
    ref = oracle.build_map(c, 3)
    kmap = _map(sp, c, 3)
    g = workloads.features(n, 64, "bf16", 521)
    for k in (13, 0, 17, 26):
        w = torch.zeros((27, 64, 64), dtype=torch.bfloat16)
        w[k] = torch.eye(64, dtype=torch.bfloat16)
        got = sp.backward_data(g.to(DEV), w.to(DEV), kmap).cpu()
        exp = torch.zeros_like(g)
        j, q = ref.lists[k]
        exp[torch.from_numpy(j).long()] = g[torch.from_numpy(q).long()]
        assert torch.equal(got, exp), f"offset {k}"
    ones_f = torch.ones((n, 32), dtype=torch.float16, device=DEV)
    ones_g = torch.ones((n, 48), dtype=torch.float16, device=DEV)
    gw = sp.backward_weights(ones_f, ones_g, kmap).cpu().numpy()
    for k in range(27):
        assert np.all(gw[k] == ref.counts[k])


@pytest.mark.parametrize("li", [0, 1])
def test_backward_batched_frames(sp, li):
    """8 batched LiDAR frames (640,812 voxels; K = 3 at C = 128 and K = 5 at
    C = 64, bf16, rows in the map's reordered row order): both gradients on
    every value.  The oracle's data gradient comes from its row-parallel
    forward over the mirrored, transposed weights (the identity pinned on
    the CPU) and its weight gradient from the offset-parallel variant."""
    layer = workloads.make_workload(4).layers[li]
    c, K = layer.coords, layer.k
    ref = oracle.build_map(c, K)
    kmap = _map(sp, c, K)
    f = workloads.features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
    g = workloads.features(layer.n, layer.cout, layer.dtype, layer.feat_seed + 7)
    w = workloads.weights(K, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
    gin = sp.backward_data(g.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    wm = np.ascontiguousarray(w.double().numpy()[::-1].transpose(0, 2, 1))
    _check_dgrad(gin, ref.forward_parallel(g.double().numpy(), wm), layer.dtype)
    gw = sp.backward_weights(f.to(DEV), g.to(DEV), kmap).double().cpu().numpy()
    fd, gd = f.double().numpy(), g.double().numpy()
    _check_wgrad(gw, ref.backward_weights_parallel(fd, gd), ref.backward_weights_parallel(np.abs(fd), np.abs(gd)))
