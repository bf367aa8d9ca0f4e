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
reported beside it.  ``roofline`` describes the fused forward kernel measured
with HIP events on the stream it runs on (recorded on about ten of the timed
steps); ``cpu_baseline`` times the CPU oracle on the host.
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
DEFAULT_WORKLOAD = 1  # the indoor scene: 150k voxels, K=3, C=32, fp16
PERMUTATION_SEED = 7  # the random row order of the permuted pass

ELEM = {"f32": 4, "f16": 2, "bf16": 2}


def algorithmic_forward_bytes(n, e, kv, cin, cout, dtype):
    """Minimum HBM bytes of one forward: each input row read once, each output
    row written once, the weights once, and the int32 input row index of every
    non-centre entry once (the output row of an entry is implied by its
    position in the output-ordered lists)."""
    s = ELEM[dtype]
    return n * cin * s + n * cout * s + kv * cin * cout * s + 4 * (e - n)


FORWARD_SOURCES = ("forward.hip",)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_forward_small_indoor_c32_f16_hbm_traffic.md")


def forward_source_digest():
    """sha256 of the source file of the small-channel forward kernel."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "submanifold_sparse_convolution_device_amd", "csrc")
    for name in FORWARD_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, _, val = line[2:].partition(": ")
            fields[key.strip("` ")] = val.strip("` ")
    try:
        if fields["forward_source_sha256"] != forward_source_digest():
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


def cpu_baseline(layer, feats, w, budget_s=12.0, max_passes=200):
    """The oracle, as it stands, on the same workload: map build (ordered-tree
    lookups) plus fp64 forward, single-threaded, repeated until ~budget_s."""
    import oracle

    fd, wd = feats.double().numpy(), w.double().numpy()
    times = []
    e = 0
    while len(times) < max_passes and sum(times) < budget_s:
        t0 = time.perf_counter()
        m = oracle.build_map(layer.coords, layer.k)
        m.forward(fd, wd)
        times.append(time.perf_counter() - t0)
        e = m.total_entries
    t = sum(times) / len(times)
    return {
        "value": 2.0 * e * layer.cin * layer.cout / t / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"whole workload (map build + fp64 forward), {len(times)} pass(es), "
                  f"{t:.2f} s per pass",
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD,
                    help="workload index 0..4 (default: the indoor scene)")
    ap.add_argument("--layer", type=int, default=0, help="layer of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    import numpy as np
    import torch

    import submanifold_sparse_convolution_device_amd as sp
    import workloads

    sp.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
    wl = workloads.make_workload(args.workload)
    layer = wl.layers[args.layer]
    feats_h, w_h = workloads.layer_inputs(layer)
    coords = torch.from_numpy(layer.coords).to(dev)
    feats = feats_h.to(dev)
    w = w_h.to(dev)
    out = torch.empty((layer.n, layer.cout), dtype=feats.dtype, device=dev)
    print(f"[bench] workload={wl.name} layer={args.layer} N={layer.n} K={layer.k} "
          f"C={layer.cin}->{layer.cout} {layer.dtype}", file=sys.stderr, flush=True)

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

    for _ in range(args.warmup):
        e_total = retire(step())
    torch.cuda.synchronize()
    kv = layer.k ** 3

    # HIP events on a sample of the timed steps (about ten, evenly spread):
    # an event record costs host and device time of its own, so timing every
    # step would slow the steps it measures.
    stride = max(1, args.steps // 10)
    sampled = list(range(0, args.steps, stride))
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    prev = None
    for i in range(args.steps):
        kmap = step(events.get(i))
        if prev is not None:
            assert retire(prev) == e_total
        prev = kmap
    assert retire(prev) == e_total
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    build_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events.values()]))
    fwd_ms = float(np.mean([ev[1].elapsed_time(ev[2]) for ev in events.values()]))

    flops = 2.0 * e_total * layer.cin * layer.cout
    value = flops / (ms_step * 1e-3) / 1e12
    fwd_bytes = algorithmic_forward_bytes(layer.n, e_total, kv, layer.cin, layer.cout, layer.dtype)
    achieved = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    result = {
        "metric": "sparse-conv effective TFLOP/s (2*|map|*Cin*Cout/t) + map build Mvoxel/s",
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": layer.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "n_voxels": layer.n,
            "map_entries": e_total,
            "kernel": layer.k,
            "c_in": layer.cin,
            "c_out": layer.cout,
        },
        "map_build_mvoxel_per_s": round(layer.n / (build_ms * 1e-3) / 1e6, 2),
        "map_build_ms": round(build_ms, 4),
        "forward_ms": round(fwd_ms, 4),
        "forward_tflops": round(flops / (fwd_ms * 1e-3) / 1e12, 4),
        "roofline": {
            "kernel": "k_forward_small (fused gather-MFMA-accumulate)" if layer.cin <= 32
                      else "k_forward_wide / k_forward_tiled (fused gather-MFMA-accumulate)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic() if (args.workload, args.layer) == (DEFAULT_WORKLOAD, 0) else None,
            "algorithmic_bytes_per_launch": int(fwd_bytes),
        },
    }
    # The same steps with two frames in flight: step i on stream i mod 2, each
    # stream retiring its own previous map, no waits between the streams.
    # The library keeps its workspaces per stream, so the two run
    # independently and one stream's latency-bound kernels share the GPU with
    # the other's.  Reported beside the single-stream figures, which `value`
    # and the roofline keep (a kernel timed while another stream runs would
    # not describe the kernel).
    if not args.no_two_streams:
        result["two_streams"] = two_stream_throughput(torch, sp, coords, feats, w, layer, args.steps,
                                                      args.warmup, e_total, flops)
    if not args.no_permuted:
        result["permuted_rows"] = permuted_throughput(torch, sp, layer, feats_h, w, args.steps, args.warmup,
                                                      e_total, flops)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layer, feats_h, w_h)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
