"""GPU parity of the backward through the C ABI against the oracle.

Data gradient: in the feature dtype, held to the forward's bound
(|gpu - oracle| <= tol x RMS(oracle) + half an ulp of the oracle's value,
tol = 2e-2 for fp16/bf16 and 1e-5 for fp32).

Weight gradient: fp32 output of sums of exactly representable products of
the stored inputs (fp16 x fp16 and bf16 x bf16 products fit fp32; fp32
inputs go through fused multiply-adds).  The library sums each offset's
entries per range of output tiles, in steps of 32 entries (one MFMA each,
or 32 fused multiply-adds in a running sum on the generic path), and then
adds the ranges in order.  Any such nested sum has a rounding error of at
most h unit roundoffs (plus second order) times the sum of the terms'
magnitudes, h being the number of roundings along the longest path from a
product to the result: 31 inside an MFMA, one per step of a range, up to 3
between the waves of a workgroup, and one per range in the final sum (on
the generic path, one per fused multiply-add instead of the first two).
_wgrad_rel derives h from the cut: ranges of ceil(tiles / ranges) 64-row
tiles, ranges = min(tiles, max(1, 2048 // (K^3 x column groups))), at most
64 entries per tile and offset.  Each value is checked against
(h + 2) x 2^-24 x sum_e |f[j_e][ci]| |g[q_e][co]|, that sum coming from the
oracle run on |f| and |g|.
"""
import numpy as np
import pytest
import torch

import box_map
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
UNIT_ROUNDOFF = 2.0 ** -24
TILE_ROWS = 64
WGRAD_UNITS = 2048


def _wgrad_rel(n, K, cin, cout, dtype):
    """Relative rounding bound of the weight gradient (see the module
    docstring): (h + 2) unit roundoffs."""
    kv = K ** 3
    cols = next((c for c in (128, 64, 32) if cout % c == 0), 16)
    mfma = (dtype != "f32" and cin in (16, 32, 64, 128, 256) and cout % 16 == 0
            and not (cin == 256 and cols == 16))
    if not mfma:
        cols = cout
        while cin * cols > 64 * 256:
            cols = (cols + 1) // 2
    groups = -(-cout // cols)
    tiles = max(1, -(-n // TILE_ROWS))
    ranges = min(tiles, max(1, WGRAD_UNITS // (kv * groups)))
    tpc = -(-tiles // ranges)
    ranges = -(-tiles // tpc)
    steps = -(-tpc * TILE_ROWS // 32)
    h = (31 + steps + 3 if mfma else 32 * steps) + ranges
    return (h + 2) * UNIT_ROUNDOFF


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


def _check_wgrad(got, ref, bound_terms, rel):
    diff = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    bound = rel * bound_terms
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
    _check_wgrad(gw, ref.backward_weights(fd, gd), ref.backward_weights(np.abs(fd), np.abs(gd)),
                 _wgrad_rel(n, K, cin, cout, dtype))


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
    _check_wgrad(gw, ref.backward_weights_parallel(fd, gd), ref.backward_weights_parallel(np.abs(fd), np.abs(gd)),
                 _wgrad_rel(layer.n, K, layer.cin, layer.cout, layer.dtype))


@pytest.mark.parametrize("boxes", [
    [(0, (256, 256, 255)), (1, (1, 16, 4095))],  # 16,777,200 rows: 2^32 - 4096 bytes at C = 128
    [(0, (256, 256, 256))]])                     # 16 rows more: the generic kernel
def test_wgrad_source_bytes_limit(sp, boxes):
    """The MFMA weight gradient addresses features and gradients with 32-bit
    byte offsets (a row past a range wraps to an offset past their end); at
    C = 128 fp16 the first case's sources fill the largest buffers it takes,
    so the last rows sit just below 2^32 bytes, and the second case runs on
    the generic kernel.  Channel 0 of row p is 1 where p mod 1024 = 1023
    (else 0, as are the other channels) and the gradient is all ones, so
    grad_W[k][0][co] counts offset k's entries (p, q) with p mod 1024 = 1023
    and every other value is 0: exact in fp32, from the boxes' closed-form
    lists."""
    K, c = 3, 128
    n = sum(lz * ly * lx for _, (lz, ly, lx) in boxes)
    kmap = sp.build_map(box_map.box_rows(boxes, DEV), K)
    f = torch.zeros((n, c), dtype=torch.float16, device=DEV)
    f[1023::1024, 0] = 1.0
    g = torch.ones((n, c), dtype=torch.float16, device=DEV)
    gw = sp.backward_weights(f, g, kmap)
    del f, g
    expect = torch.zeros((K ** 3, c, c), dtype=torch.float32, device=DEV)
    for k in range(K ** 3):
        p, _ = box_map.box_list(boxes, K, k, DEV)
        expect[k, 0, :] = float(int(((p % 1024) == 1023).sum()))
        del p
    assert torch.equal(gw, expect)
    kmap.free()
