"""GPU parity: the HIP path through the C ABI against the oracle.

Maps must match bit-exactly as per-offset sets (the order inside a list is
the library's choice: the map's row order, in which every list is checked to
be increasing, and which test_map_row_order pins to its definition).
Features must satisfy |gpu - oracle| <= tol x RMS(oracle) + half an ulp of
the oracle's value in the output type, element by element, with tol = 2e-2
for fp16/bf16 and 1e-5 for fp32, the oracle computing in fp64 on the exactly
widened stored inputs.  The half ulp is the storage rounding the output type
imposes on any correct result (bounded here by |value| x 2^-8 for bf16,
2^-11 for fp16, 2^-24 for fp32); without it, a bf16 output whose largest
values lie near 9 x RMS could not meet 2e-2 x RMS even when rounded exactly.
"""
import functools

import numpy as np
import pytest
import torch

import box_map
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
HALF_ULP = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}  # relative bound of a rounding to the type
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def sp():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import submanifold_sparse_convolution_device_amd as m
    m.lib()
    return m


DEV = "cuda:0"


@functools.lru_cache(maxsize=None)
def _workload(index):
    return workloads.make_workload(index)


def _gpu_map(sp, coords, K):
    return sp.build_map(torch.from_numpy(np.ascontiguousarray(coords, dtype=np.int32)).to(DEV), K)


def _gpu_lists(kmap):
    a, b = kmap.lists()
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def assert_map_equal(kmap, ref):
    """Per-offset set equality, counts and offsets, plus the ordering
    contract: the centre list holds every row once, in the map's row order,
    and every other list follows that order."""
    kv = ref.K ** 3
    assert kmap.kernel_size == ref.K and kmap.n == ref.N
    assert np.array_equal(kmap.counts, ref.counts)
    assert kmap.offsets[0] == 0 and np.array_equal(np.diff(kmap.offsets), kmap.counts)
    assert kmap.total_entries == ref.total_entries
    a, b = _gpu_lists(kmap)
    c = kv // 2
    order = b[kmap.offsets[c]:kmap.offsets[c + 1]]
    assert np.array_equal(np.sort(order), np.arange(ref.N)), "the centre list is not a permutation of the rows"
    rank = np.empty(ref.N, np.int64)
    rank[order] = np.arange(ref.N)
    for k in range(kv):
        lo, hi = kmap.offsets[k], kmap.offsets[k + 1]
        ga, gb = a[lo:hi], b[lo:hi]
        assert np.all(np.diff(rank[gb]) > 0), f"offset {k}: not in the map's row order"
        s = np.argsort(gb, kind="stable")
        ra, rb = ref.lists[k]  # the oracle's lists are ordered by output row
        assert np.array_equal(gb[s], rb) and np.array_equal(ga[s], ra), f"offset {k} differs"


def _forward_check(sp, kmap, coords, K, cin, cout, dtype, seed, ref_map=None, rows=None):
    f = workloads.features(coords.shape[0], cin, dtype, seed)
    w = workloads.weights(K, cin, cout, dtype, seed + 1)
    out = sp.forward(f.to(DEV), w.to(DEV), kmap)
    got = out.double().cpu().numpy()
    ref_map = ref_map or oracle.build_map(coords, K)
    fd, wd = f.double().numpy(), w.double().numpy()
    if rows is None:
        ref = ref_map.forward(fd, wd)
        sel = got
    else:
        ref = ref_map.forward_rows(fd, wd, rows)
        sel = got[rows]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    diff = np.abs(sel - ref)
    bound = TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref)
    assert np.all(np.isfinite(got))
    worst = int(np.argmax(diff - bound))
    assert np.all(diff <= bound), (f"|err| {diff.flat[worst]:.3e} > {TOL[dtype]} x RMS {rms:.3e} + half an ulp of "
                                   f"{abs(ref.flat[worst]):.3e} (max |err| {float(diff.max()):.3e})")
    return float(diff.max()) / rms


# ------------------------------------------------------------------ maps


def test_worked_5x5_map(sp):
    pts = [(1, 1), (2, 2), (2, 4), (3, 2), (4, 3)]
    c = np.array([[0, 0, r, col] for r, col in pts], np.int32)
    kmap = _gpu_map(sp, c, 3)
    assert_map_equal(kmap, oracle.build_map(c, 3))
    assert kmap.total_entries == 11 and int((kmap.counts > 0).sum()) == 5


@pytest.mark.parametrize("seed,extent,occ,batches,K", [
    (1, 6, 0.05, 1, 3), (2, 10, 0.2, 2, 3), (3, 9, 0.4, 1, 5), (4, 16, 0.1, 3, 3),
    (5, 8, 0.3, 1, 1), (6, 12, 0.05, 2, 5), (7, 7, 0.5, 1, 7), (8, 20, 0.15, 2, 3),
])
def test_map_random_grids(sp, seed, extent, occ, batches, K):
    c = workloads.permuted(workloads.random_grid(seed, extent, occ, batches), seed)
    assert_map_equal(_gpu_map(sp, c, K), oracle.build_map(c, K))


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 4095, 4096, 4097, 8193])
def test_map_ragged_sizes(sp, n):
    """Sizes around the 64-row tile and 4096-row chunk edges."""
    rng = np.random.default_rng(n)
    cells = rng.choice(40 ** 3, size=n, replace=False)
    c = np.stack([np.zeros(n), cells // 1600, (cells // 40) % 40, cells % 40], 1).astype(np.int32)
    assert_map_equal(_gpu_map(sp, c, 3), oracle.build_map(c, 3))


def test_map_extreme_coordinates(sp):
    """In-range extremes; neighbours past 2^16 - 1 or below 0 are misses, never wraps."""
    c = np.array([[32767, 65535, 65535, 65535], [32767, 65535, 65535, 65534], [32767, 0, 0, 0],
                  [0, 65535, 65535, 65535], [0, 0, 0, 0], [0, 0, 0, 1], [1, 0, 0, 0]], np.int32)
    assert_map_equal(_gpu_map(sp, c, 3), oracle.build_map(c, 3))
    assert_map_equal(_gpu_map(sp, c, 5), oracle.build_map(c, 5))


@pytest.mark.parametrize("layout", ["x_line", "z_column", "many_batches", "plane_stripes"])
def test_map_degenerate_layouts(sp, layout):
    """Layouts that load the hash and the occupancy map unevenly: a whole
    x line (65,536 voxels on one (b, z, y), so every occupancy run and home
    window of the line is full), a z column, 4,096 batches of 8 voxels at
    the same coordinates (keys that differ only in b), and alternate rows of
    a plane; each against the oracle, with K = 3 and 5, rows permuted."""
    if layout == "x_line":
        x = np.arange(65536)
        c = np.stack([np.zeros_like(x), np.full_like(x, 7), np.full_like(x, 9), x], 1)
    elif layout == "z_column":
        z = np.arange(0, 65536, 3)
        c = np.stack([np.zeros_like(z), z, np.full_like(z, 65535), np.zeros_like(z)], 1)
    elif layout == "many_batches":
        b = np.repeat(np.arange(4096), 8)
        i = np.tile(np.arange(8), 4096)
        c = np.stack([b, i // 4, (i // 2) % 2, i % 2], 1)
    else:
        y, x = np.meshgrid(np.arange(0, 400, 2), np.arange(300), indexing="ij")
        c = np.stack([np.zeros(y.size), np.full(y.size, 5), y.ravel(), x.ravel()], 1)
    c = workloads.permuted(np.ascontiguousarray(c, dtype=np.int32), 17)
    for K in (3, 5):
        assert_map_equal(_gpu_map(sp, c, K), oracle.build_map(c, K))


def test_map_dense_cube_closed_form(sp):
    """Fully active 100^3 cube (1M voxels): count(d) = prod (100 - |d_i|)."""
    n = 100
    ax = np.arange(n)
    z, y, x = np.meshgrid(ax, ax, ax, indexing="ij")
    c = np.stack([np.zeros(n ** 3), z.ravel(), y.ravel(), x.ravel()], 1).astype(np.int32)
    kmap = _gpu_map(sp, c, 3)
    for k in range(27):
        dz, dy, dx = oracle.offset_of(k, 3)
        assert kmap.counts[k] == (n - abs(dz)) * (n - abs(dy)) * (n - abs(dx))


@pytest.mark.parametrize("K,boxes,cin", [
    (3, [(0, (431, 431, 428)), (1, (1, 2, 15361))], 32),
    (7, [(0, (184, 184, 184)), (1, (2, 2, 7845))], 16)])
def test_map_and_forward_at_the_size_limit(sp, K, boxes, cin):
    """The largest n the ABI takes (n x K^3 just below 2^31: 79,536,430
    voxels at K = 3, 6,260,884 at K = 7), as two fully active boxes in
    separate batches.  Every entry of every list is checked against its
    closed form (box_map.py, itself checked against the oracle on small
    boxes): the entries of offset d are the rows q of each box whose q + d
    stays inside it (compared as sets).  The forward with all-ones features and
    weights gives C_in x deg(q), exact in fp16."""
    kv = K ** 3
    n = sum(lz * ly * lx for _, (lz, ly, lx) in boxes)
    assert n * kv < 2 ** 31 and n == (1 << 31) // kv - 1, "the largest accepted n"
    c = box_map.box_rows(boxes, DEV)
    kmap = sp.build_map(c, K)
    a, b = kmap.lists()
    for k in range(kv):
        p, q = box_map.box_list(boxes, K, k, DEV)
        lo, hi = int(kmap.offsets[k]), int(kmap.offsets[k + 1])
        assert kmap.counts[k] == q.numel(), f"offset {k} count"
        bs, s = torch.sort(b[lo:hi].long())  # the lists follow the map's row order; compare as sets
        assert torch.equal(bs, q) and torch.equal(a[lo:hi].long()[s], p), f"offset {k} entries"
        del bs, s
    del a, b
    f = torch.ones((n, cin), dtype=torch.float16, device=DEV)
    w = torch.ones((kv, cin, cin), dtype=torch.float16, device=DEV)
    out = sp.forward(f, w, kmap)
    deg = box_map.box_degree(boxes, K, DEV)
    assert torch.equal(out, (cin * deg).to(torch.float16)[:, None].expand(n, cin))
    kmap.free()


@pytest.mark.parametrize("boxes", [
    [(0, (256, 256, 255)), (1, (1, 16, 4095))],  # 16,777,200 rows: 2^32 - 4096 feature bytes at C = 128
    [(0, (256, 256, 256))]])                     # 16 rows more
def test_forward_wide_feature_bytes_limit(sp, boxes):
    """The wide path addresses the features with 32-bit byte offsets (a row
    without an entry wraps to an offset past their end, where the copy reads
    zeros).  At C = 128 fp16 the first case's features fill the largest
    buffer that path takes, so the last rows sit just below 2^32 bytes; the
    second is past it and runs on the next path.  Channel 0 of row p holds
    1 + p mod 7 (the other channels zero) and the weights are ones, so every
    output column of row q is the sum of 1 + p mod 7 over q's entries (exact
    in fp16), from the boxes' closed-form lists."""
    K, cin = 3, 128
    n = sum(lz * ly * lx for _, (lz, ly, lx) in boxes)
    c = box_map.box_rows(boxes, DEV)
    kmap = sp.build_map(c, K)
    rowval = torch.arange(n, device=DEV) % 7 + 1
    f = torch.zeros((n, cin), dtype=torch.float16, device=DEV)
    f[:, 0] = rowval.to(torch.float16)
    w = torch.ones((K ** 3, cin, cin), dtype=torch.float16, device=DEV)
    out = sp.forward(f, w, kmap)
    del f
    expect = torch.zeros(n, dtype=torch.int64, device=DEV)
    for k in range(K ** 3):
        p, q = box_map.box_list(boxes, K, k, DEV)
        expect.index_add_(0, q, rowval[p])
        del p, q
    assert torch.equal(out, expect.to(torch.float16)[:, None].expand(n, cin))
    kmap.free()


def test_map_device_errors(sp):
    dup = np.array([[0, 1, 2, 3], [0, 5, 5, 5], [0, 1, 2, 3]], np.int32)
    with pytest.raises(sp.SpconvError) as e:
        _gpu_map(sp, dup, 3)
    assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
    for bad in ([0, 0, 70000, 0], [0, -1, 0, 0], [40000, 0, 0, 0]):
        c = np.array([[0, 0, 0, 0], bad], np.int32)
        with pytest.raises(sp.SpconvError) as e:
            _gpu_map(sp, c, 3)
        assert e.value.name == "SPCONV_ERR_COORD_RANGE"
    # the library stays usable after device-detected errors
    ok = np.array([[0, 1, 2, 3], [0, 1, 2, 4]], np.int32)
    assert _gpu_map(sp, ok, 3).total_entries == 4


def test_async_build_matches_sync_and_defers_errors(sp):
    """The enqueue-only build gives the same map; a forward may follow before
    any host wait; device errors surface at the wait, and the map can still
    be freed."""
    c = workloads.permuted(workloads.random_grid(77, 16, 0.2, 2), 77)
    dc = torch.from_numpy(c).to(DEV)
    ref = oracle.build_map(c, 3)
    f = workloads.features(c.shape[0], 32, "f16", 5).to(DEV)
    w = workloads.weights(3, 32, 32, "f16", 6).to(DEV)
    m_sync = sp.build_map(dc, 3)
    out_sync = sp.forward(f, w, m_sync)
    maps = [sp.build_map(dc, 3, wait=False) for _ in range(3)]
    outs = [sp.forward(f, w, m) for m in maps]  # enqueued before any wait
    for m, o in zip(maps, outs):
        m.wait()
        assert_map_equal(m, ref)
        assert torch.equal(o, out_sync)
        m.free()
    dup = torch.from_numpy(np.array([[0, 1, 2, 3], [0, 5, 5, 5], [0, 1, 2, 3]], np.int32)).to(DEV)
    m = sp.build_map(dup, 3, wait=False)
    with pytest.raises(sp.SpconvError) as e:
        m.wait()
    assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
    with pytest.raises(sp.SpconvError):
        m.counts
    m.free()
    bad = torch.from_numpy(np.array([[0, 0, 0, 0], [0, 0, 70000, 0]], np.int32)).to(DEV)
    m = sp.build_map(bad, 3, wait=False)
    with pytest.raises(sp.SpconvError) as e:
        _ = m.total_entries
    assert e.value.name == "SPCONV_ERR_COORD_RANGE"
    m.free()
    # freeing a map whose build has not been waited on is fine too
    for _ in range(40):
        sp.build_map(dc, 3, wait=False).free()
    assert sp.build_map(dc, 3).total_entries == ref.total_entries


def test_ordered_builds_after_other_and_failed_builds(sp):
    """Maps in the neighbour-set row order (at least 262,144 rows) built one
    after another on the stream's reused scratch, with the same table size:
    keys a build left in the coordinate table would show up as neighbours
    that do not exist.  The 8 batched frames shifted one step along x, built
    right after the frames and again after two failed builds of the same
    size (one row twice; one coordinate out of range), match the oracle's
    map in full each time."""
    a = _workload(4).layers[0].coords
    b = a.copy()
    b[:, 3] += 1
    assert b[:, 3].max() < 65536
    ref_b = oracle.build_map(b, 3)
    _gpu_map(sp, a, 3).free()
    kb = _gpu_map(sp, b, 3)
    assert_map_equal(kb, ref_b)
    kb.free()
    dup = np.concatenate([a, a[7:8]])
    with pytest.raises(sp.SpconvError) as e:
        _gpu_map(sp, dup, 3)
    assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
    kb = _gpu_map(sp, b, 3)
    assert_map_equal(kb, ref_b)
    kb.free()
    bad = a.copy()
    bad[12345, 2] = 70000
    with pytest.raises(sp.SpconvError) as e:
        _gpu_map(sp, bad, 3)
    assert e.value.name == "SPCONV_ERR_COORD_RANGE"
    kb = _gpu_map(sp, b, 3)
    assert_map_equal(kb, ref_b)
    kb.free()


def test_map_sequence_on_one_stream(sp):
    """Builds enqueued back to back on one stream without host waits,
    growing, shrinking and changing K (so the stream's reused workspace is
    regrown and reused in prefixes of changing size), then each map against
    the oracle; one build fails (duplicates) in the middle of the sequence."""
    specs = [(21, 24, 0.3, 3), (22, 10, 0.5, 5), (23, 40, 0.25, 3), (24, 8, 0.6, 7), (25, 16, 0.4, 1),
             (26, 48, 0.3, 3), (27, 12, 0.5, 5), (28, 32, 0.2, 3)]
    grids = [workloads.permuted(workloads.random_grid(seed, ext, occ, 2), seed) for seed, ext, occ, _ in specs]
    dup = torch.from_numpy(np.array([[0, 1, 2, 3], [0, 5, 5, 5], [0, 1, 2, 3]], np.int32)).to(DEV)
    maps = []
    for i, (c, (_, _, _, K)) in enumerate(zip(grids, specs)):
        maps.append(sp.build_map(torch.from_numpy(c).to(DEV), K, wait=False))
        if i == 3:
            bad = sp.build_map(dup, 3, wait=False)
    with pytest.raises(sp.SpconvError) as e:
        bad.wait()
    assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
    bad.free()
    for m, c, (_, _, _, K) in zip(maps, grids, specs):
        m.wait()
        assert_map_equal(m, oracle.build_map(c, K))
        m.free()


def test_map_same_plan_repeated_on_one_stream(sp):
    """Builds of different voxel sets with the same n and K, back to back on
    one stream without host waits, so each reuses the workspace of the one
    before with the same layout, including the coordinate table that build
    left clear (no clearing launch then): nothing of an earlier build leaks
    into a later one (a stale key would show up as a false neighbour), also
    after a build that failed on duplicates and around a build with another
    K."""
    grids = [workloads.permuted(workloads.random_grid(seed, 40, 0.3, 2), seed) for seed in (61, 62, 63, 64)]
    n0 = min(g.shape[0] for g in grids)
    n0 -= n0 % 64 - 37 if n0 % 64 >= 37 else n0 % 64 + 27  # a ragged last tile
    sets = [np.ascontiguousarray(g[:n0]) for g in grids]
    dup = sets[0].copy()
    dup[-1] = dup[0]
    plan = [(sets[0], 3), (sets[1], 3), (dup, 3), (sets[2], 3), (sets[3], 5), (sets[0], 3), (sets[3], 3)]
    maps = [sp.build_map(torch.from_numpy(c).to(DEV), K, wait=False) for c, K in plan]
    for i, (m, (c, K)) in enumerate(zip(maps, plan)):
        if i == 2:
            with pytest.raises(sp.SpconvError) as e:
                m.wait()
            assert e.value.name == "SPCONV_ERR_DUPLICATE_COORD"
        else:
            m.wait()
            assert_map_equal(m, oracle.build_map(c, K))
        m.free()


def test_forward_on_another_stream_follows_the_build(sp):
    """A build enqueued without a host wait on one stream and a forward
    enqueued at once on another: the forward still sees the finished map."""
    c = workloads.random_grid(91, 40, 0.3, 1)
    dc = torch.from_numpy(c).to(DEV)
    f = workloads.features(c.shape[0], 32, "f16", 91).to(DEV)
    w = workloads.weights(3, 32, 32, "f16", 92).to(DEV)
    ref = sp.forward(f, w, sp.build_map(dc, 3))
    other = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        m = sp.build_map(dc, 3, wait=False)
        with torch.cuda.stream(other):
            out = sp.forward(f, w, m)
        other.synchronize()
        assert torch.equal(out, ref)
        m.wait()
        m.free()


def test_concurrent_host_threads(sp):
    """Four host threads, each with its own stream, build maps of different
    sizes and run forwards at once through the library's shared caches and
    summary-slot pools (ctypes releases the interpreter lock during each
    call); every map and output equals the single-threaded result."""
    import threading

    grids = [workloads.random_grid(80 + i, 10 + 2 * i, 0.3, 1) for i in range(4)]
    inputs, refs = [], []
    for i, c in enumerate(grids):
        dc = torch.from_numpy(c).to(DEV)
        f = workloads.features(c.shape[0], 32, "f16", 90 + i).to(DEV)
        w = workloads.weights(3, 32, 32, "f16", 95 + i).to(DEV)
        m = sp.build_map(dc, 3)
        refs.append((m.counts.copy(), [x.cpu() for x in m.lists()], sp.forward(f, w, m).cpu()))
        m.free()
        inputs.append((dc, f, w))
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            stream = torch.cuda.Stream()
            dc, f, w = inputs[i]
            with torch.cuda.stream(stream):
                for it in range(15):
                    m = sp.build_map(dc, 3, wait=(it % 2 == 0))
                    out = sp.forward(f, w, m)
                    m.wait()
                    lists = m.lists()
                    stream.synchronize()
                    counts, rl, ro = refs[i]
                    ok = (np.array_equal(m.counts, counts) and torch.equal(lists[0].cpu(), rl[0])
                          and torch.equal(lists[1].cpu(), rl[1]) and torch.equal(out.cpu(), ro))
                    m.free()
                    if not ok:
                        errors.append(f"thread {i} iteration {it}: result differs")
                        return
        except Exception as exc:  # reported below
            errors.append(f"thread {i}: {exc!r}")

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_forward_workspace_reuse_across_shapes(sp):
    """Forwards of different shapes on one stream with no host wait between
    them: the stream's forward workspace (operand-order weights, zero row,
    split partials) is regrown and reused while earlier forwards may still
    be running; every output equals the same forward run alone."""
    c = workloads.random_grid(55, 12, 0.35, 1)
    n = c.shape[0]
    kmap = _gpu_map(sp, c, 3)
    shapes = [(32, 32, "f16"), (64, 64, "bf16"), (256, 256, "bf16"), (32, 48, "f16"), (128, 128, "f16"),
              (64, 64, "bf16"), (256, 32, "bf16"), (16, 16, "f32")]
    inputs = [(workloads.features(n, ci, dt, 100 + i).to(DEV), workloads.weights(3, ci, co, dt, 200 + i).to(DEV))
              for i, (ci, co, dt) in enumerate(shapes)]
    alone = []
    for f, w in inputs:
        alone.append(sp.forward(f, w, kmap).cpu())
        torch.cuda.synchronize()
    outs = [sp.forward(f, w, kmap) for f, w in inputs for _ in range(2)]
    torch.cuda.synchronize()
    for i, ref in enumerate(alone):
        assert torch.equal(outs[2 * i].cpu(), ref) and torch.equal(outs[2 * i + 1].cpu(), ref), shapes[i]


ORDER_WINDOW, ORDER_KEY_BITS, ORDER_MIN_ROWS = 4096, 16, 262144


def _key_offsets(K):
    """Offsets whose neighbour flags make a row's order key, most
    significant first: those with every coordinate within one step of the
    centre, in index order, then the rest in index order, 16 of them."""
    kv, c = K ** 3, K ** 3 // 2
    inner, outer = [], []
    for k in range(kv):
        if k != c:
            (inner if max(abs(v) for v in oracle.offset_of(k, K)) <= 1 else outer).append(k)
    return (inner + outer)[:ORDER_KEY_BITS]


def expected_row_order(ref, K):
    """The map's row order by its definition, from the oracle's lists: for
    K > 1 and at least 262,144 rows, the rows of each window of 4,096
    consecutive rows sorted stably by their 16-bit neighbour key; otherwise
    the input order."""
    n = ref.N
    if K == 1 or n < ORDER_MIN_ROWS:
        return np.arange(n)
    key = np.zeros(n, np.uint32)
    for i, k in enumerate(_key_offsets(K)):
        key[ref.lists[k][1]] |= np.uint32(1) << np.uint32(ORDER_KEY_BITS - 1 - i)
    order = np.empty(n, np.int64)
    for s in range(0, n, ORDER_WINDOW):
        e = min(n, s + ORDER_WINDOW)
        order[s:e] = s + np.argsort(key[s:e], kind="stable")
    return order


def _tile_offset_pairs(b, offsets, kv, rank):
    """(64-row tile, offset) pairs with an entry, tiles taken over the
    positions `rank` gives the output rows."""
    total = 0
    for k in range(kv):
        total += np.unique(rank[b[offsets[k]:offsets[k + 1]]] // 64).size
    return total


@pytest.mark.parametrize("index,K,bound", [(4, 3, 0.65), (4, 5, 0.8), (1, 3, None), (0, 3, None)])
def test_map_row_order(sp, index, K, bound):
    """The map's row order (neighbour-bitmask row reordering): the centre
    list, which holds every row once in that order, equals the rows sorted
    stably by their 16-bit neighbour key within windows of 4,096 rows, as
    computed here from the oracle's lists; on the 8 batched LiDAR frames the
    order cuts the (tile, offset) pairs the forward visits to at most `bound`
    of the input order's.  The indoor scene (150,000 rows) and the sphere
    shell keep the input order."""
    layer = _workload(index).layers[0]
    c = layer.coords
    ref = oracle.build_map(c, K)
    kmap = _gpu_map(sp, c, K)
    a, b = _gpu_lists(kmap)
    n, kv = layer.n, K ** 3
    cen = kv // 2
    order = b[kmap.offsets[cen]:kmap.offsets[cen + 1]]
    assert np.array_equal(a[kmap.offsets[cen]:kmap.offsets[cen + 1]], order)
    assert np.array_equal(order, expected_row_order(ref, K))
    if bound is not None:
        rank = np.empty(n, np.int64)
        rank[order] = np.arange(n)
        ordered = _tile_offset_pairs(b, kmap.offsets, kv, rank)
        plain = _tile_offset_pairs(b, kmap.offsets, kv, np.arange(n))
        assert ordered <= bound * plain, f"(tile, offset) pairs {ordered} vs {plain} in input order"


def test_map_ordered_k7_ragged(sp):
    """An ordered map at K = 7 (343 offsets, six per lane in the tile count
    that runs inside the row-order kernel), on a cloud just above the
    ordering threshold whose last window and last group of 16 tiles are
    ragged: every list, count and offset equals the oracle's, and the row
    order equals its definition."""
    c = workloads.random_grid(91, 128, 0.14, 1)
    n = c.shape[0]
    assert n >= ORDER_MIN_ROWS and n % ORDER_WINDOW != 0 and ((n + 63) // 64) % 16 != 0
    ref = oracle.build_map(c, 7)
    kmap = _gpu_map(sp, c, 7)
    assert_map_equal(kmap, ref)
    a, b = _gpu_lists(kmap)
    cen = 343 // 2
    assert np.array_equal(b[kmap.offsets[cen]:kmap.offsets[cen + 1]], expected_row_order(ref, 7))
    kmap.free()


def test_map_deterministic(sp):
    c = workloads.permuted(workloads.random_grid(99, 30, 0.1, 2), 99)
    a1, b1 = _gpu_lists(_gpu_map(sp, c, 3))
    a2, b2 = _gpu_lists(_gpu_map(sp, c, 3))
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


# ------------------------------------------------------------------ forward


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("K,cin,cout", [(3, 16, 16), (3, 32, 32), (3, 32, 16), (3, 16, 32), (1, 32, 32),
                                        (3, 32, 48), (3, 8, 24), (5, 40, 16), (1, 64, 32),
                                        (3, 96, 136), (7, 16, 8), (5, 32, 32)])
def test_forward_random_grids(sp, dtype, K, cin, cout):
    if dtype == "f32" and (cin > 512 or cout > 512):
        pytest.skip("fp32 channels are limited to 512")
    c = workloads.permuted(workloads.random_grid(K * 100 + cin, 14, 0.2, 2), cin)
    kmap = _gpu_map(sp, c, K)
    _forward_check(sp, kmap, c, K, cin, cout, dtype, seed=cin * 7 + cout)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K,cin,cout", [(3, 64, 64), (3, 128, 128), (3, 256, 256), (5, 64, 64),
                                        (3, 128, 48), (3, 256, 16), (1, 128, 128), (5, 32, 64),
                                        (3, 64, 208), (7, 64, 32)])
def test_forward_mid_large_channels(sp, dtype, K, cin, cout):
    """Channel counts of the tiled path: whole W_d no longer fits on chip, so
    slices are staged per offset; C_in 256 splits a 64-row tile over two
    waves; ragged grids leave partial tiles and offsets absent from blocks."""
    c = workloads.permuted(workloads.random_grid(K * 31 + cin + cout, 13, 0.25, 2), cin + 1)
    kmap = _gpu_map(sp, c, K)
    _forward_check(sp, kmap, c, K, cin, cout, dtype, seed=cin * 5 + cout + K)


@pytest.mark.parametrize("dtype,cin,cout", [("bf16", 256, 256), ("f16", 128, 256), ("bf16", 64, 128)])
def test_forward_wide_large_grid_sampled(sp, dtype, cin, cout):
    """A grid of ~40k voxels: enough 64-row tiles that the wide path runs
    without splitting offsets, with every column group of a tile in one
    workgroup (C_in 256: two groups of 128 columns).  Sampled rows against
    the oracle."""
    c = workloads.random_grid(cin + cout, 48, 0.35, 1)
    kmap = _gpu_map(sp, c, 3)
    rows = np.sort(np.random.default_rng(cin).choice(c.shape[0], 600, replace=False))
    _forward_check(sp, kmap, c, 3, cin, cout, dtype, seed=cin + 3 * cout, rows=rows)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_forward_small_many_tiles_sampled(sp, dtype):
    """About 205k voxels at C = 32 (a box at 40% occupancy, about 10
    neighbours per row): more 64-row tiles than 11 per CU, so the
    small-channel kernel runs 12 tile waves per workgroup with no spare
    waves, some waves take a second tile, and tiles hold several stages of
    entries (the later ones gathered through the lists).  Sampled rows,
    including the last tile's, against the oracle."""
    c = workloads.random_grid(77, 80, 0.4, 1)
    n = c.shape[0]
    assert (n + 63) // 64 > 11 * 256
    kmap = _gpu_map(sp, c, 3)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(n, 600, replace=False), np.arange(n - 64, n)]))
    _forward_check(sp, kmap, c, 3, 32, 32, dtype, seed=77 if dtype == "f16" else 78, rows=rows)


@pytest.mark.parametrize("dtype,cin,cout", [("f16", 1024, 1024), ("bf16", 1024, 8), ("bf16", 8, 1024),
                                            ("f32", 512, 512), ("f32", 4, 512), ("f32", 512, 4)])
def test_forward_channel_limits(sp, dtype, cin, cout):
    """The largest channel counts the ABI takes (1024 in fp16/bf16, 512 in
    fp32) and the smallest (8 and 4), on a grid of a few ragged tiles."""
    c = workloads.permuted(workloads.random_grid(cin + cout, 7, 0.45, 1), 3)
    assert 64 < c.shape[0] < 256
    kmap = _gpu_map(sp, c, 3)
    _forward_check(sp, kmap, c, 3, cin, cout, dtype, seed=cin + 2 * cout)


@pytest.mark.parametrize("cin,cout", [(64, 64), (128, 128), (256, 256), (256, 32),
                                      (32, 64), (64, 48), (128, 80), (256, 48)])
@pytest.mark.parametrize("tiles", [2, 40, 130, 400])
def test_forward_wide_tile_counts(sp, cin, cout, tiles):
    """The wide kernel's launch choices across grid sizes: offsets split over
    up to 8 workgroups with a reduction (few tiles), narrower workgroups, and
    one workgroup per tile and column group (many tiles); the last four
    shapes go to the tiled kernel instead.  A clustered grid in bf16;
    sampled rows, including the last tile's, against the oracle."""
    rng = np.random.default_rng(tiles * 7 + cin)
    n_target = tiles * 64 - 5
    zyx = np.unique(np.concatenate([rng.integers(0, 24, size=(n_target, 3)),
                                    rng.integers(0, 300, size=(2 * n_target, 3))]), axis=0)
    zyx = zyx[rng.permutation(zyx.shape[0])[:n_target]]
    zyx = zyx[np.lexsort((zyx[:, 2], zyx[:, 1], zyx[:, 0]))]
    c = np.concatenate([np.zeros((n_target, 1), np.int64), zyx], 1).astype(np.int32)
    n = c.shape[0]
    assert (n + 63) // 64 == tiles
    kmap = _gpu_map(sp, c, 3)
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 300), replace=False), np.arange(max(0, n - 64), n)]))
    _forward_check(sp, kmap, c, 3, cin, cout, "bf16", seed=tiles + cin, rows=rows)


@pytest.mark.parametrize("K,dtype,cin,cout", [(7, "f16", 16, 16), (5, "bf16", 40, 24), (3, "f32", 48, 24),
                                              (5, "f32", 512, 64), (7, "bf16", 64, 32)])
@pytest.mark.parametrize("tiles", [2, 130, 400])
def test_forward_generic_tile_counts(sp, K, dtype, cin, cout, tiles):
    """The generic kernel (K = 5 and 7, channel counts that are not multiples
    of 16, fp32 beyond the small shapes) across grid sizes, on a clustered
    grid; sampled rows against the oracle."""
    rng = np.random.default_rng(tiles * 11 + K + cin)
    n_target = tiles * 64 - 9
    zyx = np.unique(np.concatenate([rng.integers(0, 20, size=(n_target, 3)),
                                    rng.integers(0, 200, size=(2 * n_target, 3))]), axis=0)
    zyx = zyx[rng.permutation(zyx.shape[0])[:n_target]]
    c = np.concatenate([np.zeros((n_target, 1), np.int64), zyx], 1).astype(np.int32)
    n = c.shape[0]
    kmap = _gpu_map(sp, c, K)
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 200), replace=False), np.arange(max(0, n - 64), n)]))
    _forward_check(sp, kmap, c, K, cin, cout, dtype, seed=tiles + cin + K, rows=rows)


@pytest.mark.parametrize("tiles", [3, 250, 700, 1300, 2600, 3100, 4000])
def test_forward_small_tile_counts(sp, tiles):
    """The small-channel kernel across tile counts that give 1 to 12 tile
    waves per workgroup, spare waves or none, and more tiles than waves
    (several rounds): a sparse field with dense 8^3 clusters, so some tiles
    are far heavier than the rest (split or shared with spares, several
    stages).  Sampled rows, including every row of the heaviest tiles and
    of the last tile, against the oracle."""
    rng = np.random.default_rng(tiles)
    n_target = tiles * 64 - 17
    n_clusters = max(1, n_target // 20000)
    ax = np.arange(8)
    z, y, x = np.meshgrid(ax, ax, ax, indexing="ij")
    cube = np.stack([z.ravel(), y.ravel(), x.ravel()], 1)
    parts = [cube + rng.integers(0, 400, size=3) for _ in range(n_clusters)]
    field = rng.integers(0, 2000, size=(2 * n_target, 3))
    zyx = np.unique(np.concatenate(parts + [field]), axis=0)
    zyx = zyx[rng.permutation(zyx.shape[0])[:n_target]]
    zyx = zyx[np.lexsort((zyx[:, 2], zyx[:, 1], zyx[:, 0]))]
    c = np.concatenate([np.zeros((zyx.shape[0], 1), np.int64), zyx], 1).astype(np.int32)
    n = c.shape[0]
    assert (n + 63) // 64 == tiles
    kmap = _gpu_map(sp, c, 3)
    ref = oracle.build_map(c, 3)
    deg = np.zeros(n, np.int64)
    for k in range(27):
        np.add.at(deg, ref.lists[k][1], 1)
    per_tile = np.add.reduceat(deg, np.arange(0, n, 64))
    heavy = np.argsort(per_tile)[-3:]
    rows = np.unique(np.concatenate([rng.choice(n, min(n, 500), replace=False), np.arange(max(0, n - 64), n)]
                                    + [np.arange(t * 64, min(n, t * 64 + 64)) for t in heavy]))
    _forward_check(sp, kmap, c, 3, 32, 32, "f16", seed=tiles, ref_map=ref, rows=rows)


@pytest.mark.parametrize("dtype,ch", [("f16", 32), ("bf16", 32), ("f32", 16), ("f16", 128),
                                      ("bf16", 256)])
@pytest.mark.parametrize("extent", [12, 20])
def test_forward_dense_block(sp, dtype, ch, extent):
    """Fully active cube: up to 26 neighbours per row, so a 64-row tile holds
    far more gathered rows than one stage batch."""
    ax = np.arange(extent)
    z, y, x = np.meshgrid(ax, ax, ax, indexing="ij")
    c = np.stack([np.zeros(extent ** 3), z.ravel(), y.ravel(), x.ravel()], 1).astype(np.int32)
    kmap = _gpu_map(sp, c, 3)
    _forward_check(sp, kmap, c, 3, ch, ch, dtype, seed=extent)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_forward_routing_is_exact(sp, dtype):
    """Identity weights route rows exactly in any dtype (one product by 1.0)."""
    c = workloads.permuted(workloads.random_grid(5, 12, 0.3, 1), 5)
    n = c.shape[0]
    kmap = _gpu_map(sp, c, 3)
    ref = oracle.build_map(c, 3)
    for ch in ((16, 48) if dtype == "f32" else (32, 48, 64, 256)):
        f = workloads.features(n, ch, dtype, 11)
        for k in (13, 0, 17, 26):
            w = torch.zeros((27, ch, ch), dtype=TORCH_DT[dtype])
            w[k] = torch.eye(ch, dtype=TORCH_DT[dtype])
            out = sp.forward(f.to(DEV), w.to(DEV), kmap).cpu()
            exp = torch.zeros_like(f)
            j, q = ref.lists[k]
            exp[torch.from_numpy(q).long()] = f[torch.from_numpy(j).long()]
            assert torch.equal(out, exp), f"offset {k}, {ch} channels"


def test_forward_rejects_overlapping_output(sp):
    """The output may share no byte with the features or the weights (other
    workgroups still read those while it is written): an in-place or
    overlapping output is INVALID_ARG and leaves the buffers untouched; an
    output right after the features in one allocation is fine."""
    c = workloads.random_grid(23, 9, 0.4, 1)
    n, ch = c.shape[0], 32
    kmap = _gpu_map(sp, c, 3)
    buf = torch.zeros((2 * n + 8, ch), dtype=torch.float16, device=DEV)
    feats = buf[:n]
    feats.copy_(workloads.features(n, ch, "f16", 23).to(DEV))
    w = workloads.weights(3, ch, ch, "f16", 24).to(DEV)
    before = buf.clone()
    for out in (feats, buf[n // 2:n // 2 + n], buf[1:n + 1]):
        with pytest.raises(sp.SpconvError) as e:
            sp.forward(feats, w, kmap, out=out)
        assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    wout = torch.empty((n, ch), dtype=torch.float16, device=DEV)
    wbuf = torch.zeros(27 * ch * ch + n * ch, dtype=torch.float16, device=DEV)
    wv = wbuf[:27 * ch * ch].view(27, ch, ch)
    wv.copy_(w)
    with pytest.raises(sp.SpconvError) as e:
        sp.forward(feats, wv, kmap, out=wbuf[27 * ch * ch - 8:27 * ch * ch - 8 + n * ch].view(n, ch))
    assert e.value.name == "SPCONV_ERR_INVALID_ARG"
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    ref = sp.forward(feats, w, kmap, out=wout)
    got = sp.forward(feats, w, kmap, out=buf[n:2 * n])
    assert torch.equal(got, ref) and torch.equal(buf[:n], before[:n])


@pytest.mark.parametrize("dtype,cin,cout", [("f16", 32, 32), ("bf16", 32, 16), ("f16", 64, 64),
                                            ("bf16", 128, 128), ("bf16", 256, 256), ("f16", 32, 48),
                                            ("bf16", 8, 24), ("f16", 40, 16)])
def test_forward_rounds_ties_to_even(sp, dtype, cin, cout):
    """Sums that fall exactly halfway between two values of the output type
    (1 + odd x half an ulp, with several signs and binades) come out rounded
    to the even neighbour in every kernel (small, wide with split offsets,
    tiled, generic; the wide kernel without splits in the next test); the
    epilogue's rule, checked exactly.
    Row 0 gets a + b from the centre and the +x offset (channel 0 only),
    row 1 gets a alone."""
    c = np.array([[0, 0, 0, 0], [0, 0, 0, 1]], np.int32)
    kmap = _gpu_map(sp, c, 3)
    tdt = TORCH_DT[dtype]
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11  # of values in [1, 2): 7 and 10 mantissa bits
    co = np.arange(cout)
    scale = np.array([1.0, -1.0, 2.0, -4.0])[co % 4]
    a = scale
    b = scale * half_ulp * (2 * ((co // 4) % 4) + 1)  # odd multiples: exact ties
    f = torch.zeros((2, cin), dtype=tdt)
    f[:, 0] = 1.0
    w = torch.zeros((27, cin, cout), dtype=tdt)
    w[13, 0] = torch.from_numpy(a).to(tdt)
    w[14, 0] = torch.from_numpy(b).to(tdt)  # offset (0, 0, +1): row 0 reads row 1
    assert torch.equal(w[13, 0].double(), torch.from_numpy(a)) and torch.equal(w[14, 0].double(), torch.from_numpy(b))
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).cpu()
    exp0 = torch.from_numpy(a + b).to(torch.float32).to(tdt)  # exact in fp32, then nearest-even
    # every sum is a tie: in units of the type's ulp at its binade it ends in exactly one half
    mbits = 7 if dtype == "bf16" else 10
    v = np.abs(a + b)
    units = v / 2.0 ** (np.floor(np.log2(v)) - mbits)
    assert np.all(units - np.floor(units) == 0.5)
    assert torch.equal(out[0], exp0), f"row 0: {out[0][:8]} vs {exp0[:8]}"
    assert torch.equal(out[1], torch.from_numpy(a).to(tdt))


@pytest.mark.parametrize("dtype,cin,cout", [("f16", 64, 64), ("bf16", 128, 128), ("f16", 128, 128),
                                            ("bf16", 256, 256), ("bf16", 256, 32)])
def test_forward_rounds_ties_to_even_unsplit(sp, dtype, cin, cout):
    """The same exact ties on a map with 16,384 more voxels, isolated (in
    another batch, 4 apart along x), so that the wide kernel has enough
    tiles to run without splitting offsets: its own epilogue rounds (the
    lanes' regrouped 16-byte stores) instead of the split reduction.  Rows 0
    and 1 as above; every isolated row, with zero features, is zero."""
    extra = 16384
    c = np.zeros((2 + extra, 4), np.int32)
    c[1, 3] = 1
    c[2:, 0] = 1
    c[2:, 3] = 4 * np.arange(extra)
    n = c.shape[0]
    assert (n + 63) // 64 >= 256
    kmap = _gpu_map(sp, c, 3)
    tdt = TORCH_DT[dtype]
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    co = np.arange(cout)
    scale = np.array([1.0, -1.0, 2.0, -4.0])[co % 4]
    a = scale
    b = scale * half_ulp * (2 * ((co // 4) % 4) + 1)
    f = torch.zeros((n, cin), dtype=tdt)
    f[:2, 0] = 1.0
    w = torch.zeros((27, cin, cout), dtype=tdt)
    w[13, 0] = torch.from_numpy(a).to(tdt)
    w[14, 0] = torch.from_numpy(b).to(tdt)
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).cpu()
    exp0 = torch.from_numpy(a + b).to(torch.float32).to(tdt)
    assert torch.equal(out[0], exp0), f"row 0: {out[0][:8]} vs {exp0[:8]}"
    assert torch.equal(out[1], torch.from_numpy(a).to(tdt))
    assert not torch.any(out[2:] != 0)


@pytest.mark.parametrize("dtype,cin,cout", [("f16", 32, 32), ("bf16", 64, 64), ("bf16", 128, 48),
                                            ("f32", 16, 16), ("f32", 48, 24)])
def test_forward_nonfinite_rows_stay_local(sp, dtype, cin, cout):
    """A NaN or an infinity in a few input rows reaches exactly the output
    rows whose neighbourhood holds those rows (lanes of other rows, padding
    and zero rows never pick it up); every other row matches the oracle."""
    c = workloads.permuted(workloads.random_grid(61, 11, 0.3, 1), 61)
    n = c.shape[0]
    kmap = _gpu_map(sp, c, 3)
    f = workloads.features(n, cin, dtype, 62)
    w = workloads.weights(3, cin, cout, dtype, 63)
    bad = np.array([3, n // 2, n - 1])
    f[bad[0], 5] = float("nan")
    f[bad[1], 0] = float("inf")
    f[bad[2], cin - 1] = float("-inf")
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    ref_map = oracle.build_map(c, 3)
    hit = np.zeros(n, bool)
    for k in range(27):
        j, q = ref_map.lists[k]
        hit[q[np.isin(j, bad)]] = True
    assert np.array_equal(~np.isfinite(out).all(axis=1), hit)
    clean = f.double().numpy()
    clean[bad] = 0.0
    ref = ref_map.forward(clean, w.double().numpy())
    rms = float(np.sqrt(np.mean(ref[~hit] ** 2)))
    assert np.all(np.abs(out[~hit] - ref[~hit]) <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref[~hit]))


@pytest.mark.parametrize("dtype,cin", [("f16", 32), ("f16", 64), ("bf16", 32), ("bf16", 128), ("f32", 16),
                                       ("f32", 48)])
def test_forward_subnormal_inputs(sp, dtype, cin):
    """Features in the subnormal range of their type (scaled by 2^-16 in
    fp16, 2^-128 in bf16 and fp32) against weights scaled up by 2^10 (2^20),
    so that the outputs are normal numbers: the products are formed, not
    flushed to zero, and the output matches the oracle on the same stored
    values within the usual tolerance."""
    c = workloads.random_grid(71, 10, 0.3, 1)
    n = c.shape[0]
    kmap = _gpu_map(sp, c, 3)
    fs, ws = (2.0 ** -16, 2.0 ** 10) if dtype == "f16" else (2.0 ** -128, 2.0 ** 20)
    tdt = TORCH_DT[dtype]
    f = (workloads.features(n, cin, "f32", 72).double() * fs).to(tdt)
    tiny = torch.finfo(tdt).tiny
    assert (f.double().abs() < tiny).double().mean() > 0.9 and (f != 0).double().mean() > 0.9
    w = (workloads.weights(3, cin, cin, "f32", 73).double() * ws).to(tdt)
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    ref = oracle.build_map(c, 3).forward(f.double().numpy(), w.double().numpy())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert rms > 100 * tiny, "the outputs are normal numbers"
    assert np.all(np.abs(out - ref) <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref))


def test_forward_all_ones_degree(sp):
    """All-ones features and weights: f_out[q][c] = Cin x deg(q), exact in fp16."""
    c = workloads.random_grid(17, 10, 0.5, 1)
    kmap = _gpu_map(sp, c, 3)
    n, ch = c.shape[0], 16
    out = sp.forward(torch.ones((n, ch), dtype=torch.float16, device=DEV),
                     torch.ones((27, ch, 8), dtype=torch.float16, device=DEV), kmap).cpu()
    ref = oracle.build_map(c, 3)
    deg = np.zeros(n)
    for k in range(27):
        np.add.at(deg, ref.lists[k][1], 1)
    assert torch.equal(out, torch.from_numpy(np.repeat((ch * deg)[:, None], 8, 1)).half())


def test_forward_single_voxel_and_isolated(sp):
    c = np.array([[0, 5, 5, 5]], np.int32)
    kmap = _gpu_map(sp, c, 3)
    _forward_check(sp, kmap, c, 3, 32, 32, "f16", seed=1)
    iso = np.array([[0, 3 * i, 3 * j, 0] for i in range(9) for j in range(9)], np.int32)
    _forward_check(sp, _gpu_map(sp, iso, 3), iso, 3, 32, 16, "bf16", seed=2)


@pytest.mark.parametrize("index,seed", [(1, None), (None, 31)])
def test_forward_small_spare_fallback(sp, monkeypatch, index, seed):
    """A spare wave of the small-channel forward that shares its owner's
    stage waits a bounded time, then gathers its half tile itself.  With the
    wait skipped (SPCONV_SMALL_SPIN_LIMIT = -1) or cut to one check (0), the
    output is bit-identical to the default one (same products, same order)
    and matches the oracle: the indoor scene (C = 32 f16, ten owner waves and
    two spares per workgroup; 2,298 of its 2,344 tiles hold 64 to 128
    non-centre entries, the range whose upper half a spare shares) and a
    random grid with shared and heavy tiles (C = 16 f32, one owner and two
    spares per workgroup)."""
    if index is not None:
        layer = _workload(index).layers[0]
        c, K, cin, cout, dtype = layer.coords, layer.k, layer.cin, layer.cout, layer.dtype
    else:
        c, K, cin, cout, dtype = workloads.random_grid(seed, 40, 0.08, 1), 3, 16, 16, "f32"
    kmap = _gpu_map(sp, c, K)
    f = workloads.features(c.shape[0], cin, dtype, 5).to(DEV)
    w = workloads.weights(K, cin, cout, dtype, 6).to(DEV)
    monkeypatch.delenv("SPCONV_SMALL_SPIN_LIMIT", raising=False)
    base = sp.forward(f, w, kmap)
    for limit in ("-1", "0"):
        monkeypatch.setenv("SPCONV_SMALL_SPIN_LIMIT", limit)
        got = sp.forward(f, w, kmap)
        torch.cuda.synchronize()
        assert torch.equal(got, base), f"limit {limit}"
    monkeypatch.delenv("SPCONV_SMALL_SPIN_LIMIT")
    ref = oracle.build_map(c, K).forward(f.double().cpu().numpy(), w.double().cpu().numpy())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    diff = np.abs(base.double().cpu().numpy() - ref)
    assert np.all(diff <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(ref))


def test_forward_is_repeatable_and_overwrites(sp):
    c = workloads.random_grid(23, 16, 0.2, 1)
    kmap = _gpu_map(sp, c, 3)
    f = workloads.features(c.shape[0], 32, "f16", 1).to(DEV)
    w = workloads.weights(3, 32, 32, "f16", 2).to(DEV)
    out = torch.full((c.shape[0], 32), float("nan"), dtype=torch.float16, device=DEV)
    a = sp.forward(f, w, kmap, out=out).clone()
    b = sp.forward(f, w, kmap)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ large layers (four-tile workgroups)


@pytest.mark.parametrize("seed,extent,occ,batches,K,cin,dtype,permute", [
    (401, 96, 0.2, 1, 3, 128, "bf16", False),   # N ~ 177k, ragged last task
    (402, 70, 0.25, 2, 3, 128, "f16", True),    # two batches, rows permuted
    (403, 80, 0.3, 1, 3, 64, "bf16", False),
    (404, 64, 0.3, 2, 5, 64, "f16", True),      # K = 5: offsets beyond 64
    (405, 62, 0.2, 3, 5, 128, "bf16", False),   # three batches, K = 5 at C = 128
])
def test_forward_large_layers(sp, seed, extent, occ, batches, K, cin, dtype, permute):
    """Layers of well over 512 four-tile tasks (the four-tile workgroup path)
    against the oracle on every output row, with sizes that leave a ragged
    last tile and task."""
    c = workloads.random_grid(seed, extent, occ, batches)
    if permute:
        c = workloads.permuted(c, seed)
    assert c.shape[0] > 512 * 256 and c.shape[0] % 256 != 0
    ref = oracle.build_map(c, K)
    kmap = _gpu_map(sp, c, K)
    f = workloads.features(c.shape[0], cin, dtype, seed + 1)
    w = workloads.weights(K, cin, cin, dtype, seed + 2)
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    r = ref.forward_parallel(f.double().numpy(), w.double().numpy())
    rms = float(np.sqrt(np.mean(r ** 2)))
    diff = np.abs(out - r)
    assert np.all(np.isfinite(out))
    assert np.all(diff <= TOL[dtype] * rms + HALF_ULP[dtype] * np.abs(r)), \
        f"max |err| {float(diff.max()):.3e} vs RMS {rms:.3e}"


@pytest.mark.parametrize("cin,K", [(128, 3), (64, 3), (64, 5)])
def test_forward_large_routing_is_exact(sp, cin, K):
    """Identity weights at one offset route rows exactly on the four-tile
    path too (centre: the task's own rows, read without an index; other
    offsets: gathered rows, with rows lacking the neighbour zeroed)."""
    c = workloads.random_grid(410 + K, 90, 0.2, 1)
    n = c.shape[0]
    assert n > 512 * 256
    kmap = _gpu_map(sp, c, K)
    ref = oracle.build_map(c, K)
    kv = K ** 3
    f = workloads.features(n, cin, "bf16", 412)
    for k in (kv // 2, 0, kv // 2 + 1, kv - 1):
        w = torch.zeros((kv, cin, cin), dtype=torch.bfloat16)
        w[k] = torch.eye(cin, dtype=torch.bfloat16)
        out = sp.forward(f.to(DEV), w.to(DEV), kmap).cpu()
        exp = torch.zeros_like(f)
        j, q = ref.lists[k]
        exp[torch.from_numpy(q).long()] = f[torch.from_numpy(j).long()]
        assert torch.equal(out, exp), f"offset {k}, {cin} channels"


# ------------------------------------------------------------------ the five workloads


@pytest.mark.parametrize("index", [0, 1, 2])
def test_workload_map_and_forward(sp, index):
    wl = _workload(index)
    layer = wl.layers[0]
    ref = oracle.build_map(layer.coords, layer.k)
    kmap = _gpu_map(sp, layer.coords, layer.k)
    assert_map_equal(kmap, ref)
    _forward_check(sp, kmap, layer.coords, layer.k, layer.cin, layer.cout, layer.dtype,
                   seed=layer.feat_seed, ref_map=ref)


def test_workload_permuted_rows(sp):
    """The bench workload (indoor scene) with its rows in the seeded random
    order of bench.py's permuted pass: whole map and whole forward against
    the oracle."""
    layer = _workload(1).layers[0]
    perm = np.random.default_rng(7).permutation(layer.n)
    c = np.ascontiguousarray(layer.coords[perm])
    ref = oracle.build_map(c, layer.k)
    kmap = _gpu_map(sp, c, layer.k)
    assert_map_equal(kmap, ref)
    _forward_check(sp, kmap, c, layer.k, layer.cin, layer.cout, layer.dtype, seed=layer.feat_seed, ref_map=ref)


def test_workload_unet_stack(sp):
    """Four levels x two chained convs; conv 2 takes conv 1's GPU output as
    stored (bf16), and the oracle takes that same tensor, so parity is per
    layer."""
    wl = _workload(3)
    prev = None
    for layer in wl.layers:
        if not layer.chain:
            ref = oracle.build_map(layer.coords, layer.k)
            kmap = _gpu_map(sp, layer.coords, layer.k)
            assert_map_equal(kmap, ref)
            f = workloads.features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
        else:
            f = prev.cpu()
        w = workloads.weights(layer.k, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
        out = sp.forward(f.to(DEV), w.to(DEV), kmap)
        r = ref.forward(f.double().numpy(), w.double().numpy())
        rms = float(np.sqrt(np.mean(r ** 2)))
        diff = np.abs(out.double().cpu().numpy() - r)
        assert np.all(diff <= TOL[layer.dtype] * rms + HALF_ULP[layer.dtype] * np.abs(r)), \
            f"level {layer.level}: {float(diff.max()):.3e} vs RMS {rms:.3e}"
        prev = out


@pytest.mark.parametrize("li", [0, 1])
def test_workload_batched_frames(sp, li):
    """8 batched LiDAR frames (640,812 voxels), K = 3 at C = 128 and K = 5 at
    C = 64, bf16: the whole map against the oracle's as per-offset sets
    (every list element, counts and offsets), and the whole forward against
    the oracle's fp64 forward on every output row (its row-parallel variant,
    pinned bit-identical to the serial one on the CPU)."""
    layer = _workload(4).layers[li]
    ref = oracle.build_map(layer.coords, layer.k)
    kmap = _gpu_map(sp, layer.coords, layer.k)
    assert_map_equal(kmap, ref)
    f = workloads.features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
    w = workloads.weights(layer.k, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
    out = sp.forward(f.to(DEV), w.to(DEV), kmap).double().cpu().numpy()
    r = ref.forward_parallel(f.double().numpy(), w.double().numpy())
    rms = float(np.sqrt(np.mean(r ** 2)))
    diff = np.abs(out - r)
    assert np.all(np.isfinite(out))
    bound = TOL[layer.dtype] * rms + HALF_ULP[layer.dtype] * np.abs(r)
    assert np.all(diff <= bound), f"max |err| {float(diff.max()):.3e} vs RMS {rms:.3e}"
