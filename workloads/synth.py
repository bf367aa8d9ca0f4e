"""Seeded synthetic voxel workloads for submanifold sparse convolution.

This module only draws inputs: integer voxel coordinates ``(b, z, y, x)``,
feature rows and weight tensors.  It holds none of the convolution's
arithmetic (no hashing, no neighbour search, no products), so both the CPU
oracle and the GPU path can consume its output without sharing any of the
method's code.

The shapes follow the pages' workload descriptions:

* "Sparse inputs and sparse convolution" (course notes), opening section:
  outdoor LiDAR frames are below 0.01 % occupied, indoor scans and single
  objects below 1 %.
* "TorchSparse: regular computation from irregular sparsity", section
  "Measured: neither zero padding nor one group wins": per-offset map sizes
  differ by an order of magnitude (thousands outdoors, hundreds on smaller
  scenes).

The public datasets those pages measure on are not available; the five
generators below stand in for them.  Every choice the workload descriptions
leave open is a stated reading (sphere radius rounding, wall height, LiDAR beam
fan, box size ranges).

All coordinates are returned as ``int32[N, 4]`` in lexicographic
``(b, z, y, x)`` order without duplicates, which is what a unique-based
voxelizer emits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Tuple

import numpy as np
import torch

# --------------------------------------------------------------------------
# coordinate generators
# --------------------------------------------------------------------------


def _lexsort_unique(bzyx: np.ndarray) -> np.ndarray:
    """Deduplicate rows of an int64 [M,4] array and sort them lexicographically."""
    if bzyx.shape[0] == 0:
        return np.zeros((0, 4), dtype=np.int32)
    u = np.unique(bzyx.astype(np.int64), axis=0)  # np.unique sorts rows lexicographically
    return np.ascontiguousarray(u.astype(np.int32))


def sphere_shell(radius: int = 20, grid: int = 64) -> np.ndarray:
    """Cells ``v`` of a ``grid^3`` box whose rounded distance to the box centre
    equals ``radius`` (batch 0).  Reading of "cells on a sphere surface of
    radius 20 centred in a 64^3 grid"."""
    c = grid // 2
    ax = np.arange(grid, dtype=np.float64)
    z, y, x = np.meshgrid(ax, ax, ax, indexing="ij")
    d = np.sqrt((z - c) ** 2 + (y - c) ** 2 + (x - c) ** 2)
    sel = np.rint(d) == radius
    zz, yy, xx = z[sel].astype(np.int64), y[sel].astype(np.int64), x[sel].astype(np.int64)
    b = np.zeros_like(zz)
    return _lexsort_unique(np.stack([b, zz, yy, xx], axis=1))


def indoor_scene(seed: int, n_keep: int = 150_000, grid: int = 512,
                 wall_height: int = 160, n_boxes: int = 20) -> np.ndarray:
    """Floor plane, four walls and ``n_boxes`` axis-aligned boxes standing on the
    floor, surfaces voxelized one voxel thick, deduplicated, then a uniform
    random subset of ``n_keep`` voxels (batch 0).

    Readings: wall height 160 voxels; box sides drawn from U{16..96} per axis;
    the five visible faces of each box (not the one resting on the floor) are
    voxelized."""
    rng = np.random.default_rng(seed)
    parts = []
    g = grid
    # floor z = 0
    yy, xx = np.meshgrid(np.arange(g), np.arange(g), indexing="ij")
    parts.append(np.stack([np.zeros(g * g), yy.ravel(), xx.ravel()], axis=1))
    # walls x in {0, g-1} and y in {0, g-1}, z in [0, wall_height)
    zz, tt = np.meshgrid(np.arange(wall_height), np.arange(g), indexing="ij")
    zz, tt = zz.ravel(), tt.ravel()
    for fixed in (0, g - 1):
        parts.append(np.stack([zz, tt, np.full_like(tt, fixed)], axis=1))   # x = fixed
        parts.append(np.stack([zz, np.full_like(tt, fixed), tt], axis=1))   # y = fixed
    # boxes
    for _ in range(n_boxes):
        sx, sy, sz = (int(v) for v in rng.integers(16, 97, size=3))
        x0 = int(rng.integers(1, g - 1 - sx))
        y0 = int(rng.integers(1, g - 1 - sy))
        x1, y1, z1 = x0 + sx - 1, y0 + sy - 1, sz - 1
        xs, ys, zs = np.arange(x0, x1 + 1), np.arange(y0, y1 + 1), np.arange(0, z1 + 1)
        # top face z = z1
        a, b_ = np.meshgrid(ys, xs, indexing="ij")
        parts.append(np.stack([np.full(a.size, z1), a.ravel(), b_.ravel()], axis=1))
        # faces x = x0 and x = x1
        a, b_ = np.meshgrid(zs, ys, indexing="ij")
        for xf in (x0, x1):
            parts.append(np.stack([a.ravel(), b_.ravel(), np.full(a.size, xf)], axis=1))
        # faces y = y0 and y = y1
        a, b_ = np.meshgrid(zs, xs, indexing="ij")
        for yf in (y0, y1):
            parts.append(np.stack([a.ravel(), np.full(a.size, yf), b_.ravel()], axis=1))
    zyx = np.concatenate(parts, axis=0).astype(np.int64)
    zyx = np.unique(zyx, axis=0)
    keep = rng.choice(zyx.shape[0], size=min(n_keep, zyx.shape[0]), replace=False)
    zyx = zyx[keep]
    b = np.zeros((zyx.shape[0], 1), dtype=np.int64)
    return _lexsort_unique(np.concatenate([b, zyx], axis=1))


def lidar_frame(seed: int, batch: int = 0, beams: int = 64, azimuths: int = 2048,
                n_boxes: int = 40, voxel: float = 0.1) -> np.ndarray:
    """One ray-cast LiDAR-like frame: a sensor at height 1.8 m casts
    ``beams x azimuths`` rays onto a ground plane and ``n_boxes`` axis-aligned
    boxes standing on it; the first hit of each ray is voxelized at ``voxel`` m
    into a 2048 x 2048 x 256 grid spanning x, y in [-102.4, 102.4) m and
    z in [-2.0, 23.6) m.

    Readings: beam elevations linspace(-5 deg, +5 deg, beams); box centre at a
    radius drawn from U(20, 95) m and an azimuth from U(0, 2 pi); footprint sides
    and heights from U(4, 20) m; no range noise."""
    rng = np.random.default_rng(seed)
    el = np.deg2rad(np.linspace(-5.0, 5.0, beams))
    az = 2.0 * np.pi * np.arange(azimuths) / azimuths
    E, A = np.meshgrid(el, az, indexing="ij")
    d = np.stack([np.cos(E) * np.cos(A), np.cos(E) * np.sin(A), np.sin(E)], axis=-1).reshape(-1, 3)
    o = np.array([0.0, 0.0, 1.8])
    t_best = np.full(d.shape[0], np.inf)
    # ground plane z = 0 (only rays pointing down reach it)
    down = d[:, 2] < 0
    t_best[down] = -o[2] / d[down, 2]
    # boxes
    r = rng.uniform(20.0, 95.0, n_boxes)
    phi = rng.uniform(0.0, 2.0 * np.pi, n_boxes)
    sx = rng.uniform(4.0, 20.0, n_boxes)
    sy = rng.uniform(4.0, 20.0, n_boxes)
    h = rng.uniform(4.0, 20.0, n_boxes)
    cx, cy = r * np.cos(phi), r * np.sin(phi)
    lo = np.stack([cx - sx / 2, cy - sy / 2, np.zeros(n_boxes)], axis=1)
    hi = np.stack([cx + sx / 2, cy + sy / 2, h], axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = 1.0 / d  # inf where a direction component is 0
        for i in range(n_boxes):
            t1 = (lo[i] - o) * inv
            t2 = (hi[i] - o) * inv
            tmin = np.nanmax(np.minimum(t1, t2), axis=1)
            tmax = np.nanmin(np.maximum(t1, t2), axis=1)
            hit = (tmax >= np.maximum(tmin, 0.0)) & (tmin > 0.0)
            t_best = np.where(hit & (tmin < t_best), tmin, t_best)
    ok = np.isfinite(t_best)
    p = o + d[ok] * t_best[ok, None]
    ix = np.floor((p[:, 0] + 102.4) / voxel).astype(np.int64)
    iy = np.floor((p[:, 1] + 102.4) / voxel).astype(np.int64)
    iz = np.floor((p[:, 2] + 2.0) / voxel).astype(np.int64)
    inr = (ix >= 0) & (ix < 2048) & (iy >= 0) & (iy < 2048) & (iz >= 0) & (iz < 256)
    bzyx = np.stack([np.full(int(inr.sum()), batch), iz[inr], iy[inr], ix[inr]], axis=1)
    return _lexsort_unique(bzyx)


def coarsen(coords: np.ndarray) -> np.ndarray:
    """Next level of a U-Net-like pyramid: ``unique((b, z//2, y//2, x//2))``,
    the outputs of a K = 2, stride 2 strided map of the level (the library's
    strided map produces the same coordinates; the tests check it)."""
    c = coords.astype(np.int64).copy()
    c[:, 1:] //= 2
    return _lexsort_unique(c)


def batched_lidar(seeds=tuple(range(100, 108))) -> np.ndarray:
    """Independent LiDAR frames concatenated, frame i carrying batch index i."""
    frames = [lidar_frame(s, batch=i) for i, s in enumerate(seeds)]
    return np.ascontiguousarray(np.concatenate(frames, axis=0))


# --------------------------------------------------------------------------
# features and weights
# --------------------------------------------------------------------------

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def features(n: int, c: int, dtype: str, seed: int) -> torch.Tensor:
    """Feature rows drawn from N(0, 1) in float64, rounded (RNE) to ``dtype``."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((n, c))
    return torch.from_numpy(f).to(_TORCH_DTYPES[dtype]).contiguous()


def weights(k: int, cin: int, cout: int, dtype: str, seed: int) -> torch.Tensor:
    """Weights ``[k^3, cin, cout]`` drawn from N(0, 1/(k^3 cin)) (the second
    parameter read as the variance, a fan-in scaling) in float64, rounded to
    ``dtype``."""
    rng = np.random.default_rng(seed)
    kv = k ** 3
    w = rng.standard_normal((kv, cin, cout)) / math.sqrt(kv * cin)
    return torch.from_numpy(w).to(_TORCH_DTYPES[dtype]).contiguous()


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Layer:
    """One submanifold convolution over ``coords``: kernel ``k``, channels
    ``cin -> cout`` in ``dtype``.  ``chain`` marks a layer whose input is the
    previous layer's output (same coordinates, same map)."""
    coords: np.ndarray
    k: int
    cin: int
    cout: int
    dtype: str
    feat_seed: int
    weight_seed: int
    level: int = 0
    chain: bool = False

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])


@dataclasses.dataclass
class Workload:
    name: str
    description: str
    layers: List[Layer]


WORKLOAD_NAMES = (
    "sphere_shell_c16_f32",
    "indoor_c32_f16",
    "lidar_c64_f16",
    "lidar_unet4_bf16",
    "lidar_batch8_bf16",
)


def make_workload(index: int) -> Workload:
    """Workload ``index`` in 0..4 (the five configurations, in order)."""
    base = 1000 * (index + 1)
    if index == 0:
        c = sphere_shell()
        return Workload(WORKLOAD_NAMES[0],
                        "sphere shell r=20 in 64^3, K=3, C=16, fp32",
                        [Layer(c, 3, 16, 16, "f32", base + 100, base + 200)])
    if index == 1:
        c = indoor_scene(seed=base + 0)
        return Workload(WORKLOAD_NAMES[1],
                        "indoor scene 512^3, 150k voxels, K=3, C=32, fp16",
                        [Layer(c, 3, 32, 32, "f16", base + 100, base + 200)])
    if index == 2:
        c = lidar_frame(seed=3)
        return Workload(WORKLOAD_NAMES[2],
                        "LiDAR frame 64x2048 rays, K=3, C=64, fp16",
                        [Layer(c, 3, 64, 64, "f16", base + 100, base + 200)])
    if index == 3:
        layers = []
        c = lidar_frame(seed=3)
        for lvl, ch in enumerate((32, 64, 128, 256)):
            if lvl > 0:
                c = coarsen(c)
            layers.append(Layer(c, 3, ch, ch, "bf16", base + 100 + lvl, base + 200 + 2 * lvl, lvl, False))
            layers.append(Layer(c, 3, ch, ch, "bf16", base + 100 + lvl, base + 201 + 2 * lvl, lvl, True))
        return Workload(WORKLOAD_NAMES[3],
                        "LiDAR U-Net stack: 4 levels x 2 convs, C=32..256, bf16", layers)
    if index == 4:
        c = batched_lidar()
        return Workload(WORKLOAD_NAMES[4],
                        "8 LiDAR frames batched, K=3 C=128 and K=5 C=64, bf16",
                        [Layer(c, 3, 128, 128, "bf16", base + 100, base + 200),
                         Layer(c, 5, 64, 64, "bf16", base + 101, base + 201)])
    raise ValueError(f"workload index {index} out of range 0..4")


def layer_inputs(layer: Layer) -> Tuple[torch.Tensor, torch.Tensor]:
    """(features, weights) of ``layer`` as CPU tensors in the layer's dtype."""
    f = features(layer.n, layer.cin, layer.dtype, layer.feat_seed)
    w = weights(layer.k, layer.cin, layer.cout, layer.dtype, layer.weight_seed)
    return f, w


# --------------------------------------------------------------------------
# small random sets for property and edge-case tests
# --------------------------------------------------------------------------


def random_grid(seed: int, extent: int, occupancy: float, batches: int = 1,
                dims: int = 3) -> np.ndarray:
    """Random subset of an ``extent^dims`` box (per batch) at ``occupancy``,
    embedded as (b, z, y, x) with unused leading axes set to 0."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(batches):
        m = rng.random((extent,) * dims) < occupancy
        idx = np.argwhere(m)
        pad = np.zeros((idx.shape[0], 3 - dims), dtype=np.int64)
        rows.append(np.concatenate([np.full((idx.shape[0], 1), b), pad, idx], axis=1))
    return _lexsort_unique(np.concatenate(rows, axis=0)) if rows else np.zeros((0, 4), np.int32)


def permuted(coords: np.ndarray, seed: int) -> np.ndarray:
    """The same voxel set with its rows in a seeded random order."""
    rng = np.random.default_rng(seed)
    return np.ascontiguousarray(coords[rng.permutation(coords.shape[0])])
