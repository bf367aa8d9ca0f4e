"""Benchmark of the submanifold sparse convolution hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the kernel-map build (hash insert, half-offset probe with mirror emission,
per-offset scan and compaction) followed by the fused forward (centre GEMM,
gathered offsets on MFMA, output-stationary accumulation, epilogue).  Inputs
are resident in HBM before timing starts.

Steps are pipelined the way a network would run them: each map build is
enqueued without a host wait, the forward follows on the same stream, and the
previous step's map is waited on (its device status checked) and released
once this step's work is queued.

Prints ONE JSON line.  ``value`` is the whole-step effective throughput
2 |map| C_in C_out / t_step in TFLOP/s (|map| counts real entries only,
including the centre ones); the map-build rate and the forward-only rate are
reported beside it, with the forward alone timed per call and with its
weights prepared once (spconv_weights_prepare: the weight re-layout out of
the call).  ``roofline`` describes the fused forward kernel measured
with HIP events on the stream it runs on (recorded on about ten of the timed
steps); ``cpu_baseline`` times the CPU oracle on the host.  Beside the step,
the line reports the two gradients, the strided convolution and its
transpose, and the weight-stationary grouped dataflow (gather, batched
products, reduction) against the fused forward with the library's
per-layer dataflow selector.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
# The largest configuration that fits one GPU: 8 batched LiDAR frames
# (640,812 voxels), K=3, C=128, bf16.  Its K=5 C=64 layer, the indoor
# scene (150k voxels, K=3, C=32, fp16) and the U-Net stack's C=256 layer
# (4,789 voxels, bf16) are timed the same way and reported beside it in the
# same line.
DEFAULT_WORKLOAD = 4
DEFAULT_LAYER = 0
EXTRA_LAYERS = ((4, 1), (1, 0), (3, 6))
PERMUTATION_SEED = 7  # the random row order of the permuted pass

ELEM = {"f32": 4, "f16": 2, "bf16": 2}


def algorithmic_forward_bytes(n, e, kv, cin, cout, dtype):
    """Minimum HBM bytes of one forward: each input row read once, each output
    row written once, the weights once, and 8 bytes (an int32 input and output
    row index) per non-centre entry of the map."""
    s = ELEM[dtype]
    return n * cin * s + n * cout * s + kv * cin * cout * s + 8 * (e - n)


def roofline(layer, e, fwd_ms, traffic=None):
    """Roofline of one forward: the ceiling is min(MFMA peak, AI x HBM peak)
    with AI = 2 E C_in C_out / algorithmic bytes; `bound` names the side that
    sets it, and `achieved`/`peak`/`frac` are in that side's unit.  Both
    fractions are reported beside it."""
    kv = layer.k ** 3
    nbytes = algorithmic_forward_bytes(layer.n, e, kv, layer.cin, layer.cout, layer.dtype)
    return roofline_of(2.0 * e * layer.cin * layer.cout, nbytes, fwd_ms, layer.dtype, traffic)


def strided_forward_bytes(n_in, n_out, e, kv, cin, cout, dtype):
    """Minimum HBM bytes of a forward over a strided or transposed map: the
    input rows read once, the output rows written once, the weights once and
    8 bytes of row indices per entry (no entry is an identity)."""
    s = 4 if dtype == "f32" else 2
    return n_in * cin * s + n_out * cout * s + kv * cin * cout * s + 8 * e


def roofline_of(flops, nbytes, fwd_ms, dtype, traffic=None):
    ai = flops / nbytes
    t = fwd_ms * 1e-3
    gbs = nbytes / t / 1e9
    tflops = flops / t / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS[dtype]
    hbm_frac = gbs / HBM_PEAK_GBS
    mfma_frac = tflops / mfma_peak
    mfma_bound = mfma_peak * 1e12 < ai * HBM_PEAK_GBS * 1e9
    r = {
        "bound": "mfma" if mfma_bound else "hbm",
        "achieved": round(tflops if mfma_bound else gbs, 2),
        "peak": mfma_peak if mfma_bound else HBM_PEAK_GBS,
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "frac": round(mfma_frac if mfma_bound else hbm_frac, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": int(nbytes),
        "flops_per_launch": int(flops),
        "arithmetic_intensity": round(ai, 1),
        "hbm_frac": round(hbm_frac, 4),
        "mfma_frac": round(mfma_frac, 4),
        "time_at_roofline_us": round(max(flops / (mfma_peak * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)) * 1e6, 2),
    }
    return r


# Counter summaries of HBM traffic per forward launch, by (workload, layer):
# the profile and the kernel sources whose sha256 it was taken on.
TRAFFIC_PROFILES = {
    (4, 0): ("k_forward_wide_batch8_k3_c128_bf16_hbm_traffic.md", ("forward_wide.hip", "forward_tiled.hip")),
    (4, 1): ("k_forward_wide_batch8_k5_c64_bf16_hbm_traffic.md", ("forward_wide.hip", "forward_tiled.hip")),
    (1, 0): ("k_forward_small_indoor_c32_f16_hbm_traffic.md", ("forward.hip",)),
}


def source_digest(names):
    """sha256 over the named kernel source files, in order."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "submanifold_sparse_convolution_device_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload, layer):
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none or the kernel sources changed since it was taken."""
    entry = TRAFFIC_PROFILES.get((workload, layer))
    if entry is None:
        return None
    name, sources = entry
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, _, val = line[2:].partition(": ")
            fields[key.strip("` ")] = val.strip("` ")
    try:
        if fields["forward_source_sha256"] != source_digest(sources):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, dev, mib=256, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM
    counters: FETCH_SIZE and WRITE_SIZE of this copy should each read `mib`
    MiB per dispatch."""
    src = torch.ones(mib * 2**20 // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def host_cpu():
    """(logical CPUs, model name) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count() or 0, model


def cpu_baseline(layer, feats, w, leg_s=8.0):
    """The oracle, as it stands, timed on the host on a bounded sample of the
    same workload, in two legs:
      * all cores: the map build (single-threaded ordered-tree lookups) plus
        the fp64 forward split over output rows on every host thread, over
        the whole voxel set;
      * one core: the map build plus the serial fp64 forward, over the first
        frame of the batch (batch index 0) when there are several, else the
        whole set.
    Each leg's value is 2 |map| C_in C_out / t over what it ran, t being the
    mean of passes repeated for about leg_s seconds."""
    import numpy as np
    import oracle

    nproc, model = host_cpu()
    threads = oracle.max_threads()
    fd, wd = feats.double().numpy(), w.double().numpy()

    # Each leg repeats its pass until it has run about `leg_s` seconds.
    t_all, passes_all = 0.0, 0
    t_build = 0.0
    while passes_all == 0 or t_all < leg_s:
        t0 = time.perf_counter()
        m = oracle.build_map(layer.coords, layer.k)
        t1 = time.perf_counter()
        m.forward_parallel(fd, wd, threads)
        t2 = time.perf_counter()
        t_build += t1 - t0
        t_all += t2 - t0
        passes_all += 1
        e_all = m.total_entries
        del m
    t_build /= passes_all
    t_all /= passes_all

    c = layer.coords
    sel = c[:, 0] == c[0, 0]
    one_frame = bool(sel.sum() < c.shape[0])
    idx = np.nonzero(sel)[0]
    t_one, passes_one = 0.0, 0
    while passes_one == 0 or t_one < leg_s:
        t0 = time.perf_counter()
        m1 = oracle.build_map(c[idx], layer.k)
        m1.forward(fd[idx], wd)
        t_one += time.perf_counter() - t0
        passes_one += 1
        e_one = m1.total_entries
        del m1
    t_one /= passes_one
    flop = 2.0 * layer.cin * layer.cout
    return {
        "value": round(flop * e_all / t_all / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole workload ({layer.n} voxels, {e_all} entries): map build {t_build:.2f} s "
                  f"single-threaded + fp64 forward on {threads} threads, {t_all:.2f} s per pass, "
                  f"{passes_all} pass(es)",
        "nproc": nproc,
        "cpu_model": model,
        "single_core": {
            "value": round(flop * e_one / t_one / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": 1,
            "sample": (f"first frame of the batch ({idx.shape[0]} voxels, {e_one} entries)" if one_frame
                       else f"whole workload ({e_one} entries)")
            + f": map build + serial fp64 forward, {t_one:.2f} s per pass, {passes_one} pass(es)",
        },
    }


def two_stream_throughput(torch, sp, coords, feats, w, layer, steps, warmup, e_total, flops):
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = [torch.empty((layer.n, layer.cout), dtype=feats.dtype, device=feats.device) for _ in streams]
    prev = [None, None]

    def run(count):
        for i in range(count):
            j = i % 2
            with torch.cuda.stream(streams[j]):
                kmap = sp.build_map(coords, layer.k, wait=False)
                sp.forward(feats, w, kmap, out=outs[j])
                if prev[j] is not None:
                    prev[j].wait()
                    assert prev[j].total_entries == e_total
                    prev[j].free()
                prev[j] = kmap

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    for j in range(2):
        if prev[j] is not None:
            with torch.cuda.stream(streams[j]):
                prev[j].wait()
                assert prev[j].total_entries == e_total
                prev[j].free()
            prev[j] = None
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": round(ms, 4), "value": round(flops / (ms * 1e-3) / 1e12, 4), "unit": "TFLOP/s",
            "note": "the same steps, two frames in flight on two streams (steady-state throughput)"}


def permuted_throughput(torch, sp, layer, feats_h, w, steps, warmup, e_total, flops):
    """The same single-stream steps with the workload's rows in a seeded
    random order (coordinates and features permuted together): the map and
    the output are the same up to that relabelling, but neighbouring rows no
    longer sit in neighbouring lanes, so loads and stores stop coalescing."""
    import numpy as np

    perm = np.random.default_rng(PERMUTATION_SEED).permutation(layer.n)
    dev = w.device
    coords = torch.from_numpy(np.ascontiguousarray(layer.coords[perm])).to(dev)
    feats = feats_h[torch.from_numpy(perm)].contiguous().to(dev)
    out = torch.empty((layer.n, layer.cout), dtype=feats.dtype, device=dev)

    def run(count):
        prev = None
        for _ in range(count):
            kmap = sp.build_map(coords, layer.k, wait=False)
            sp.forward(feats, w, kmap, out=out)
            if prev is not None:
                prev.wait()
                assert prev.total_entries == e_total
                prev.free()
            prev = kmap
        prev.wait()
        assert prev.total_entries == e_total
        prev.free()

    run(max(1, warmup))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": round(ms, 4), "value": round(flops / (ms * 1e-3) / 1e12, 4), "unit": "TFLOP/s",
            "note": f"the same steps with the rows in a seeded random order (seed {PERMUTATION_SEED})"}


def measure(torch, sp, layer, steps, warmup, events_wanted=10):
    """Single-stream steps over `layer`; returns the step time and the mean
    build and forward times from HIP events on the launch stream."""
    import numpy as np

    dev = torch.device("cuda:0")
    feats_h, w_h = _inputs(layer)
    coords = torch.from_numpy(layer.coords).to(dev)
    feats = feats_h.to(dev)
    w = w_h.to(dev)
    out = torch.empty((layer.n, layer.cout), dtype=feats.dtype, device=dev)

    # One step: the map build, enqueued without a host wait, then the forward
    # on the same stream.  The previous step's map is waited on (its device
    # status checked) and released after this step's work is enqueued, so the
    # device never idles between steps and every map is still checked.
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        kmap = sp.build_map(coords, layer.k, wait=False)
        if ev is not None:
            ev[1].record()
        sp.forward(feats, w, kmap, out=out)
        if ev is not None:
            ev[2].record()
        return kmap

    def retire(kmap):
        kmap.wait()  # raises on a device-detected build error
        e = kmap.total_entries
        kmap.free()  # stream-ordered release, as a network layer would do
        return e

    e_total = None
    for _ in range(max(1, warmup)):
        e_total = retire(step())
    torch.cuda.synchronize()

    # HIP events on a sample of the timed steps (about ten, evenly spread):
    # an event record costs host and device time of its own, so timing every
    # step would slow the steps it measures.
    stride = max(1, steps // events_wanted)
    sampled = list(range(0, steps, stride))
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    prev = None
    for i in range(steps):
        kmap = step(events.get(i))
        if prev is not None:
            assert retire(prev) == e_total
        prev = kmap
    assert retire(prev) == e_total
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # The whole synchronous build call (kernels and the one summary read-back)
    # by the host clock, median of ten after the steps above warmed it.
    calls = []
    for _ in range(10):
        c0 = time.perf_counter()
        kmap = sp.build_map(coords, layer.k)
        calls.append((time.perf_counter() - c0) * 1e3)
        kmap.free()
    torch.cuda.synchronize()
    # The forward alone on one map, as called per step (weights re-laid out
    # in the call) and with weights prepared once (spconv_weights_prepare):
    # HIP event pairs, the two taking turns in rounds of 10 (so that clock
    # drift meets both alike), median of 40 each.
    kmap = sp.build_map(coords, layer.k)
    pw = sp.prepare_weights(w)
    fwd = {"call": lambda: sp.forward(feats, w, kmap, out=out),
           "prepared": lambda: sp.forward_prepared(feats, pw, kmap, out=out)}
    times = {name: [] for name in fwd}
    for rnd in range(4):
        for name, fn in fwd.items():
            for _ in range(2):
                fn()
            for _ in range(10):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                b.synchronize()
                times[name].append(a.elapsed_time(b))
    alone = {name: float(np.median(ts)) for name, ts in times.items()}
    pw.free()
    kmap.free()
    torch.cuda.synchronize()
    return {
        "fwd_call_ms": alone["call"], "fwd_prepared_ms": alone["prepared"],
        "build_call_ms": float(np.median(calls)),
        "ms_step": (t1 - t0) * 1e3 / steps,
        "build_ms": float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events.values()])),
        "fwd_ms": float(np.mean([ev[1].elapsed_time(ev[2]) for ev in events.values()])),
        "e_total": e_total,
        "coords": coords, "feats": feats, "w": w, "feats_h": feats_h, "w_h": w_h,
    }


def build_roofline(n, e, k, build_ms):
    """Roofline of one map build by the survey's byte model per voxel: 16
    (coordinates) + 12 (insert: key and value) + 12 per probe of the
    (K^3 - 1) / 2 half offsets + 8 per non-centre entry written; beside it
    the line-granular bound, a 64-byte line per random probe.  Integer work:
    the ceiling is HBM bandwidth."""
    half = (k ** 3 - 1) // 2
    per_voxel = 16 + 12 + 12 * half + 8 * (e / n - 1)
    per_voxel_lines = 16 + 12 + 64 * half + 8 * (e / n - 1)
    t = build_ms * 1e-3
    gbs = n * per_voxel / t / 1e9
    return {
        "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_voxel": round(per_voxel, 1),
        "frac_line_granular": round(n * per_voxel_lines / t / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_voxel_line_granular": round(per_voxel_lines, 1),
        "time_at_roofline_us": round(n * per_voxel / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
    }


def measure_ceilings(torch, reps=10):
    """The chip's ceilings as measured here: a 1 GiB device-to-device copy
    (read + write bytes per second) and a dense 8192^3 bf16 matrix product
    (PyTorch's library GEMM), each the median of `reps` HIP event pairs."""
    import numpy as np

    dev = torch.device("cuda:0")

    def events(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    src = torch.empty(1 << 29, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    t_copy = events(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    x = torch.randn((m, m), device=dev).to(torch.bfloat16)
    y = torch.randn((m, m), device=dev).to(torch.bfloat16)
    t_mm = events(lambda: torch.matmul(x, y))
    del x, y
    return {
        "hbm_copy_gbs": round(2 * (1 << 30) / (t_copy * 1e-3) / 1e9, 1),
        "bf16_gemm_tflops": round(2 * m ** 3 / (t_mm * 1e-3) / 1e12, 1),
        "note": "device copy of 1 GiB (read + write) and an 8192^3 bf16 GEMM, median of HIP event pairs",
    }


def measure_backward(torch, sp, layer, reps=20, warmup=3):
    """Both gradients of the forward over one map of `layer`, each timed
    with HIP events on the launch stream (median of `reps`): the data
    gradient (the forward over the mirrored, transposed weights, its
    weight re-layout kernel included) and the weight gradient (gather-gather
    MFMA sums per offset and their chunk reduction)."""
    import numpy as np
    import workloads

    dev = torch.device("cuda:0")
    f, w = _inputs(layer)
    g = workloads.features(layer.n, layer.cout, layer.dtype, layer.feat_seed + 7)
    coords = torch.from_numpy(layer.coords).to(dev)
    f, w, g = f.to(dev), w.to(dev), g.to(dev)
    kmap = sp.build_map(coords, layer.k)
    gin = torch.empty_like(f)
    gw = torch.empty((layer.k ** 3, layer.cin, layer.cout), dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_data = timed(lambda: sp.backward_data(g, w, kmap, out=gin))
    t_w = timed(lambda: sp.backward_weights(f, g, kmap, out=gw))
    e = kmap.total_entries
    kmap.free()
    flops = 2.0 * e * layer.cin * layer.cout
    return {
        "data_gradient_ms": round(t_data, 4),
        "data_gradient_tflops": round(flops / (t_data * 1e-3) / 1e12, 2),
        "data_gradient_roofline": roofline(layer, e, t_data),
        "weight_gradient_ms": round(t_w, 4),
        "weight_gradient_tflops": round(flops / (t_w * 1e-3) / 1e12, 2),
        "weight_gradient_mfma_frac": round(flops / (t_w * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[layer.dtype], 4),
        "note": "one map, median of HIP event pairs; weight gradient written in fp32",
    }


def measure_strided(torch, sp, coords_np, K=3, stride=2, cin=64, cout=128, dtype="bf16", reps=10):
    """The strided (downsampling) convolution between pyramid levels and its
    transpose (upsampling back), on the given coordinates: map builds (host
    wall time of the call, which waits for the device; median of `reps`) and
    forwards (HIP event pairs on the launch stream, median of `reps`)."""
    import numpy as np
    import workloads

    dev = torch.device("cuda:0")
    coords = torch.from_numpy(coords_np).to(dev)
    torch.cuda.synchronize()

    def wall(fn):
        # two untimed calls first; each new map replaces (and frees) the last
        ts, res = [], None
        for _ in range(reps + 2):
            res = None
            t0 = time.perf_counter()
            res = fn()
            torch.cuda.synchronize()
            ts.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(ts[2:])), res

    def events(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_build, kmap = wall(lambda: sp.build_map_strided(coords, K, stride))
    t_tr, tmap = wall(kmap.transpose)
    f = workloads.features(kmap.n_in, cin, dtype, 900).to(dev)
    w = workloads.weights(K, cin, cout, dtype, 901).to(dev)
    out = torch.empty((kmap.n, cout), dtype=f.dtype, device=dev)
    t_down = events(lambda: sp.forward(f, w, kmap, out=out))
    g = workloads.features(kmap.n, cout, dtype, 902).to(dev)
    wt = workloads.weights(K, cout, cin, dtype, 903).to(dev)
    up = torch.empty((kmap.n_in, cin), dtype=f.dtype, device=dev)
    t_up = events(lambda: sp.forward(g, wt, tmap, out=up))
    e = kmap.total_entries
    kv = K ** 3
    res = {
        "kernel": K, "stride": stride, "n_in": int(kmap.n_in), "n_out": int(kmap.n), "map_entries": int(e),
        "c_in": cin, "c_out": cout, "dtype": dtype,
        "map_build_ms": round(t_build, 4), "transpose_build_ms": round(t_tr, 4),
        "down_forward_ms": round(t_down, 4),
        "down_roofline": roofline_of(2.0 * e * cin * cout,
                                     strided_forward_bytes(kmap.n_in, kmap.n, e, kv, cin, cout, dtype), t_down, dtype),
        "up_forward_ms": round(t_up, 4),
        "up_roofline": roofline_of(2.0 * e * cin * cout,
                                   strided_forward_bytes(kmap.n, kmap.n_in, e, kv, cout, cin, dtype), t_up, dtype),
        "note": "map builds: host wall time of the call (it waits for the device twice); forwards: HIP event pairs",
    }
    tmap.free()
    kmap.free()
    return res


def grouped_dataflow_bytes(n, e, padded, kv, cin, cout, dtype):
    """Minimum HBM bytes of the gather-GEMM-scatter dataflow with padded
    batches: the gather reads each entry's input row (and its 4-byte index)
    and writes the padded batch; the batched products read the batch and the
    weights and write one fp32 product row per entry; the reduction reads
    those and writes each output row once."""
    s = ELEM[dtype]
    gather = e * cin * s + 4 * e + padded * cin * s
    gemm = padded * cin * s + kv * cin * cout * s + e * cout * 4
    reduce = e * cout * 4 + n * cout * s
    return gather + gemm + reduce


# Plans of the grouped dataflow timed beside the fused forward:
# (label, epsilon, S).
DATAFLOW_PLANS = (("dense", 1.0, float("inf")), ("symmetric", 0.0, float("inf")),
                  ("adaptive", 0.2, float("inf")), ("separate", 0.0, 0.0))
DATAFLOW_LAYERS = ((4, 0), (1, 0), (3, 6))


def measure_dataflows(torch, sp, cases, reps=10):
    """Fused forward against the weight-stationary grouped dataflow on each
    (workload, layer): HIP event pairs on the launch stream (median of
    `reps`) for the fused forward and each plan of DATAFLOW_PLANS, then the
    library's selector over its default (epsilon, S) grid.  The roofline of
    the fastest grouped plan is taken against that dataflow's own bytes
    (grouped_dataflow_bytes) and its executed (padded) products."""
    import numpy as np
    import workloads

    dev = torch.device("cuda:0")

    def events(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    out_rows = []
    for wi, li in cases:
        wl = workloads.make_workload(wi)
        layer = wl.layers[li]
        print(f"[bench] dataflows: workload={wl.name} layer={li} N={layer.n} K={layer.k} "
              f"C={layer.cin}->{layer.cout} {layer.dtype}", file=sys.stderr, flush=True)
        f, w = _inputs(layer)
        f, w = f.to(dev), w.to(dev)
        kmap = sp.build_map(torch.from_numpy(layer.coords).to(dev), layer.k)
        out = torch.empty((layer.n, layer.cout), dtype=f.dtype, device=dev)
        e = kmap.total_entries
        kv = layer.k ** 3
        row = {"workload": wl.name, "layer": li, "n_voxels": layer.n, "map_entries": int(e), "kernel": layer.k,
               "c_in": layer.cin, "c_out": layer.cout, "dtype": layer.dtype,
               "fused_ms": round(events(lambda: sp.forward(f, w, kmap, out=out)), 4)}
        best = None
        for label, eps, S in DATAFLOW_PLANS:
            groups, padded = sp.group_plan(kmap, eps, S)
            t = events(lambda: sp.forward_grouped(f, w, kmap, eps, S, out=out))
            row[label] = {"epsilon": eps, "S": S if np.isfinite(S) else "inf", "groups": len(groups),
                          "padded_rows": int(padded), "ms": round(t, 4)}
            if best is None or t < best[0]:
                best = (t, label, padded)
        t, label, padded = best
        row["grouped_best"] = label
        row["grouped_best_roofline"] = roofline_of(
            2.0 * padded * layer.cin * layer.cout,
            grouped_dataflow_bytes(layer.n, e, padded, kv, layer.cin, layer.cout, layer.dtype), t, layer.dtype)
        row["fused_speedup_over_best_grouped"] = round(t / row["fused_ms"], 2)
        choice, _ = sp.select_dataflow(f, w, kmap, reps=3, out=out)
        row["selector"] = {k: (v if not isinstance(v, float) or np.isfinite(v) else "inf")
                           for k, v in choice.items()}
        kmap.free()
        out_rows.append(row)
    return out_rows


def _inputs(layer):
    import workloads

    return workloads.layer_inputs(layer)


def layer_summary(wl, layer, li, r, traffic):
    flops = 2.0 * r["e_total"] * layer.cin * layer.cout
    return {
        "workload": wl.name,
        "layer": li,
        "n_voxels": layer.n,
        "map_entries": r["e_total"],
        "kernel": layer.k,
        "c_in": layer.cin,
        "c_out": layer.cout,
        "dtype": layer.dtype,
        "ms_per_step": round(r["ms_step"], 4),
        "value": round(flops / (r["ms_step"] * 1e-3) / 1e12, 4),
        "map_build_ms": round(r["build_ms"], 4),
        "map_build_mvoxel_per_s": round(layer.n / (r["build_ms"] * 1e-3) / 1e6, 2),
        "map_build_call_ms": round(r["build_call_ms"], 4),
        "map_build_roofline": build_roofline(layer.n, r["e_total"], layer.k, r["build_ms"]),
        "forward_ms": round(r["fwd_ms"], 4),
        "forward_tflops": round(flops / (r["fwd_ms"] * 1e-3) / 1e12, 4),
        "forward_alone_ms": round(r["fwd_call_ms"], 4),
        "forward_prepared_ms": round(r["fwd_prepared_ms"], 4),
        "forward_prepared_tflops": round(flops / (r["fwd_prepared_ms"] * 1e-3) / 1e12, 4),
        "roofline": roofline(layer, r["e_total"], r["fwd_ms"], traffic),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD,
                    help="workload index 0..4 (default: the 8 batched LiDAR frames)")
    ap.add_argument("--layer", type=int, default=DEFAULT_LAYER, help="layer of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip measuring the copy and GEMM ceilings")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra layers reported beside the default one")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the two gradients")
    ap.add_argument("--no-strided", action="store_true", help="skip timing the strided convolution")
    ap.add_argument("--no-dataflows", action="store_true",
                    help="skip timing the grouped weight-stationary dataflow against the fused forward")
    ap.add_argument("--no-permuted", action="store_true",
                    help="skip the pass over the rows in a random order")
    ap.add_argument("--no-two-streams", action="store_true",
                    help="skip the two-stream throughput pass (e.g. when tracing kernel durations)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 256 MiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path; the workload would shard by frame, one frame set per GPU",
              file=sys.stderr)
        return 2

    import torch

    import submanifold_sparse_convolution_device_amd as sp
    import workloads

    sp.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
    wl = workloads.make_workload(args.workload)
    layer = wl.layers[args.layer]
    print(f"[bench] workload={wl.name} layer={args.layer} N={layer.n} K={layer.k} "
          f"C={layer.cin}->{layer.cout} {layer.dtype}", file=sys.stderr, flush=True)
    r = measure(torch, sp, layer, args.steps, args.warmup)
    e_total = r["e_total"]
    summary = layer_summary(wl, layer, args.layer, r, recorded_traffic(args.workload, args.layer))
    flops = 2.0 * e_total * layer.cin * layer.cout
    rl = dict(summary["roofline"])
    rl["kernel"] = ("k_forward_small (fused gather-MFMA-accumulate)" if layer.cin <= 32
                    else "k_forward_wide / k_forward_tiled (fused gather-MFMA-accumulate; the forward "
                         "call, whose weight re-layout kernel is included)")
    result = {
        "metric": "sparse-conv effective TFLOP/s (2*|map|*Cin*Cout/t) + map build Mvoxel/s",
        "value": summary["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summary["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": layer.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "layer": args.layer,
            "n_voxels": layer.n,
            "map_entries": e_total,
            "kernel": layer.k,
            "c_in": layer.cin,
            "c_out": layer.cout,
        },
        "map_build_mvoxel_per_s": summary["map_build_mvoxel_per_s"],
        "map_build_ms": summary["map_build_ms"],
        "map_build_call_ms": summary["map_build_call_ms"],
        "map_build_roofline": summary["map_build_roofline"],
        "forward_ms": summary["forward_ms"],
        "forward_tflops": summary["forward_tflops"],
        "forward_alone_ms": summary["forward_alone_ms"],
        "forward_prepared_ms": summary["forward_prepared_ms"],
        "forward_prepared_tflops": summary["forward_prepared_tflops"],
        "roofline": rl,
    }
    # The same steps with two frames in flight: step i on stream i mod 2, each
    # stream retiring its own previous map, no waits between the streams.
    # The library keeps its workspaces per stream, so the two run
    # independently and one stream's latency-bound kernels share the GPU with
    # the other's.  Reported beside the single-stream figures, which `value`
    # and the roofline keep (a kernel timed while another stream runs would
    # not describe the kernel).
    if not args.no_two_streams:
        result["two_streams"] = two_stream_throughput(torch, sp, r["coords"], r["feats"], r["w"], layer,
                                                      args.steps, args.warmup, e_total, flops)
    if not args.no_permuted:
        result["permuted_rows"] = permuted_throughput(torch, sp, layer, r["feats_h"], r["w"], args.steps,
                                                      args.warmup, e_total, flops)
    main_inputs = (r["feats_h"], r["w_h"])
    del r
    if not args.no_backward:
        result["backward"] = measure_backward(torch, sp, layer)
    if not args.no_strided:
        result["strided"] = measure_strided(torch, sp, layer.coords)
    if not args.no_dataflows:
        result["dataflows"] = measure_dataflows(torch, sp, DATAFLOW_LAYERS)
    if not args.no_extra and (args.workload, args.layer) == (DEFAULT_WORKLOAD, DEFAULT_LAYER):
        extra = []
        for wi, li in EXTRA_LAYERS:
            xwl = wl if wi == args.workload else workloads.make_workload(wi)
            xl = xwl.layers[li]
            print(f"[bench] extra: workload={xwl.name} layer={li} N={xl.n} K={xl.k} "
                  f"C={xl.cin}->{xl.cout} {xl.dtype}", file=sys.stderr, flush=True)
            xr = measure(torch, sp, xl, args.steps, args.warmup)
            extra.append(layer_summary(xwl, xl, li, xr, recorded_traffic(wi, li)))
            del xr
        result["other_layers"] = extra
    if not args.no_ceilings:
        c = measure_ceilings(torch)
        fwd_s = summary["forward_ms"] * 1e-3
        nbytes = rl["algorithmic_bytes_per_launch"]
        c["forward_frac_of_measured"] = round(min(
            1.0, max(flops / fwd_s / 1e12 / c["bf16_gemm_tflops"], nbytes / fwd_s / 1e9 / c["hbm_copy_gbs"])), 4) \
            if layer.dtype != "f32" else None
        c["forward_mfma_frac_of_measured"] = round(flops / fwd_s / 1e12 / c["bf16_gemm_tflops"], 4)
        c["forward_hbm_frac_of_measured"] = round(nbytes / fwd_s / 1e9 / c["hbm_copy_gbs"], 4)
        result["ceilings_measured"] = c
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layer, *main_inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
