"""The no-allocation forward (spconv_forward_noalloc) against spconv_forward.

The variant runs the same kernels with the library's fixed per-device scratch
in place of the stream's allocated workspace, so its output must equal
spconv_forward's bit for bit; both are also held to the oracle's tolerance.
Two calls in a row, the second on a smaller input (so that stale scratch
contents from the first would show), then a third shape that splits its
offsets (fp32 partials in the scratch), and a shape whose workspace exceeds
the scratch (rejected before any launch)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
HALF_ULP = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


def _case(sp, seed, extent, occ, batches, K, cin, cout, dtype):
    c = workloads.permuted(workloads.random_grid(seed, extent, occ, batches), seed)
    n = c.shape[0]
    kmap = sp.build_map(torch.from_numpy(c).to(DEV), K)
    f = workloads.features(n, cin, dtype, seed + 1)
    w = workloads.weights(K, cin, cout, dtype, seed + 2)
    fd, wd = f.to(DEV), w.to(DEV)
    out_na = torch.full((n, cout), float("nan"), dtype=TORCH_DT[dtype], device=DEV)
    sp.forward(fd, wd, kmap, out=out_na, noalloc=True)
    ref_gpu = sp.forward(fd, wd, kmap)
    torch.cuda.synchronize()
    print(f"[no_alloc] seed={seed} N={n} K={K} C={cin}->{cout} {dtype}", flush=True)
    assert torch.equal(out_na, ref_gpu), "noalloc output differs from spconv_forward's"
    r = oracle.build_map(c, K).forward(f.double().numpy(), w.double().numpy())
    rms = float(np.sqrt(np.mean(r ** 2)))
    got = out_na.double().cpu().numpy()
    assert np.all(np.abs(got - r) <= 2e-2 * rms + HALF_ULP[dtype] * np.abs(r))
    kmap.free()
    return n


def test_noalloc_matches_forward_twice_then_smaller(sp):
    n1 = _case(sp, 301, 40, 0.12, 2, 3, 128, 128, "bf16")   # wide path, many tiles
    n2 = _case(sp, 302, 14, 0.25, 1, 3, 64, 64, "f16")      # smaller input, split offsets
    assert n2 < n1
    n3 = _case(sp, 303, 10, 0.3, 1, 3, 32, 48, "f16")       # tiled path
    assert n3 < n2
    _case(sp, 304, 8, 0.3, 1, 3, 256, 256, "bf16")          # C = 256, split offsets


def test_noalloc_rejects_workspace_beyond_scratch(sp):
    """Weights of 125 x 256 x 1024 bf16 (64 MiB in operand order) exceed the
    32 MiB scratch: UNSUPPORTED, nothing launched, the output untouched."""
    c = workloads.random_grid(305, 6, 0.3, 1)
    n = c.shape[0]
    kmap = sp.build_map(torch.from_numpy(c).to(DEV), 5)
    f = workloads.features(n, 256, "bf16", 306).to(DEV)
    w = torch.zeros((125, 256, 1024), dtype=torch.bfloat16, device=DEV)
    out = torch.full((n, 1024), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sp.SpconvError) as e:
        sp.forward(f, w, kmap, out=out, noalloc=True)
    assert e.value.name == "SPCONV_ERR_UNSUPPORTED"
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    kmap.free()
