"""GPU checks of the forward with prepared weights (spconv_weights_prepare,
spconv_forward_prepared) through the C ABI.

The prepared forward is the same computation as spconv_forward with the
weights the handle copied, so its output must equal spconv_forward's bit for
bit on every path (small, wide with and without split offsets, tiled,
generic, strided and transposed maps); one case is also compared with the
oracle's fp64 forward within the forward's bound.  The handle is a snapshot:
writing the source tensor afterwards changes nothing, and one handle serves
several maps of its kernel volume.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


def _coords(c):
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV)


def _inputs(n_in, K, cin, cout, dtype, seed):
    f = workloads.features(n_in, cin, dtype, seed).to(DEV)
    w = workloads.weights(K, cin, cout, dtype, seed + 1).to(DEV)
    return f, w


# (grid extent, occupancy, K, C_in, C_out, dtype): small-channel, wide at
# three widths (the C_in = 256 layer small enough to split its offsets),
# tiled, K = 5 and the generic fp32 path.
CASES = [
    (40, 0.1, 3, 32, 32, "f16"),
    (48, 0.3, 3, 64, 64, "bf16"),
    (48, 0.3, 3, 128, 128, "bf16"),
    (20, 0.3, 3, 256, 256, "bf16"),
    (30, 0.2, 3, 32, 64, "f16"),
    (24, 0.2, 5, 64, 128, "f16"),
    (24, 0.2, 3, 16, 24, "f32"),
]


@pytest.mark.parametrize("extent,occ,K,cin,cout,dtype", CASES)
def test_prepared_equals_forward(sp, extent, occ, K, cin, cout, dtype):
    c = workloads.random_grid(extent * 7 + cin + cout, extent, occ, 2)
    kmap = sp.build_map(_coords(c), K)
    f, w = _inputs(c.shape[0], K, cin, cout, dtype, seed=extent + cin)
    ref = sp.forward(f, w, kmap)
    pw = sp.prepare_weights(w)
    got = sp.forward_prepared(f, pw, kmap)
    again = sp.forward_prepared(f, pw, kmap, out=torch.full_like(got, 7))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(again, ref)
    pw.free()
    kmap.free()


@pytest.mark.parametrize("K,stride,cin,cout", [(2, 2, 64, 64), (3, 2, 128, 64)])
def test_prepared_strided_and_transposed(sp, K, stride, cin, cout):
    c = workloads.random_grid(K * 100 + cin, 40, 0.2, 2)
    down = sp.build_map_strided(_coords(c), K, stride)
    up = down.transpose()
    f, w = _inputs(c.shape[0], K, cin, cout, "bf16", seed=K + cin)
    pw = sp.prepare_weights(w)
    y = sp.forward(f, w, down)
    assert torch.equal(sp.forward_prepared(f, pw, down), y)
    w2 = workloads.weights(K, cout, cin, "bf16", 5).to(DEV)
    pw2 = sp.prepare_weights(w2)
    assert torch.equal(sp.forward_prepared(y, pw2, up), sp.forward(y, w2, up))
    pw.free()
    pw2.free()
    up.free()
    down.free()


def test_prepared_against_oracle(sp):
    """The prepared wide path against the oracle's fp64 forward."""
    K, cin, cout, dtype = 3, 128, 128, "bf16"
    c = workloads.random_grid(11, 40, 0.3, 1)
    kmap = sp.build_map(_coords(c), K)
    f, w = _inputs(c.shape[0], K, cin, cout, dtype, seed=3)
    pw = sp.prepare_weights(w)
    got = sp.forward_prepared(f, pw, kmap).double().cpu().numpy()
    ref = oracle.build_map(c, K).forward(f.double().cpu().numpy(), w.double().cpu().numpy())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(got - ref) <= 2e-2 * rms + 2.0 ** -8 * np.abs(ref))
    pw.free()
    kmap.free()


def test_prepared_is_a_snapshot_and_serves_several_maps(sp):
    K, cin, cout, dtype = 3, 64, 64, "f16"
    f_seed = 21
    c1 = workloads.random_grid(1, 36, 0.3, 1)
    c2 = workloads.random_grid(2, 30, 0.25, 2)
    m1, m2 = sp.build_map(_coords(c1), K), sp.build_map(_coords(c2), K)
    f1, w = _inputs(c1.shape[0], K, cin, cout, dtype, seed=f_seed)
    f2 = workloads.features(c2.shape[0], cin, dtype, f_seed + 5).to(DEV)
    ref1, ref2 = sp.forward(f1, w, m1), sp.forward(f2, w, m2)
    pw = sp.prepare_weights(w)
    w.mul_(-3)  # after the copy was enqueued on the same stream
    assert torch.equal(sp.forward_prepared(f1, pw, m1), ref1)
    assert torch.equal(sp.forward_prepared(f2, pw, m2), ref2)
    assert not torch.equal(sp.forward(f1, w, m1), ref1)
    pw.free()
    m1.free()
    m2.free()


def test_prepared_rejects_mismatches(sp):
    c = workloads.random_grid(4, 20, 0.3, 1)
    m3 = sp.build_map(_coords(c), 3)
    w5 = workloads.weights(5, 32, 32, "f16", 1).to(DEV)
    pw5 = sp.prepare_weights(w5)
    f = workloads.features(c.shape[0], 32, "f16", 2).to(DEV)
    with pytest.raises(sp.SpconvError):
        sp.forward_prepared(f, pw5, m3)
    # the raw entry point checks the kernel volume itself
    out = torch.empty((c.shape[0], 32), dtype=torch.float16, device=DEV)
    with pytest.raises(sp.SpconvError) as e:
        sp.spconv_forward_prepared(f.data_ptr(), pw5.handle, m3.handle, out.data_ptr(), 0)
    assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    assert "offsets" in sp.spconv_last_error()
    pw5.free()
    pw5.free()  # a second free is a no-op
    m3.free()
