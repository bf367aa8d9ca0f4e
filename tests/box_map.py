"""Closed forms for the maps of fully active boxes, used to check the
library at sizes the oracle cannot reach (tests only; pinned against the
oracle on small boxes in test_box_map.py).

A box is (b, (Lz, Ly, Lx)): every voxel (b, z, y, x) with 0 <= z < Lz,
0 <= y < Ly, 0 <= x < Lx, in lexicographic (z, y, x) order; boxes follow one
another in the row order and sit in different batches, so no entry joins
two of them (entries never cross b).  For an offset d, Q + d stays inside
Q's box exactly on the sub-box max(0, -d_a) <= v_a < L_a - max(0, d_a) of
each axis a, so offset d's list, ordered by output row, is that sub-box in
lexicographic order, box after box, with P = Q + d.
"""
from typing import List, Sequence, Tuple

import torch

Box = Tuple[int, Tuple[int, int, int]]


def box_rows(boxes: Sequence[Box], dev) -> torch.Tensor:
    """int32 [N, 4] (b, z, y, x) of the boxes, in row order."""
    parts = []
    for b, (lz, ly, lx) in boxes:
        q = torch.arange(lz * ly * lx, device=dev, dtype=torch.int64)
        parts.append(torch.stack([torch.full_like(q, b), q // (lx * ly), (q // lx) % ly, q % lx], 1))
    return torch.cat(parts).to(torch.int32).contiguous()


def offset_of(k: int, K: int) -> Tuple[int, int, int]:
    """(dz, dy, dx) of offset index k = ((dz + r) K + (dy + r)) K + (dx + r)."""
    r = (K - 1) // 2
    return (k // (K * K) - r, (k // K) % K - r, k % K - r)


def box_list(boxes: Sequence[Box], K: int, k: int, dev) -> Tuple[torch.Tensor, torch.Tensor]:
    """(in rows P, out rows Q) of offset k, int64, ordered by Q."""
    d = offset_of(k, K)
    ps: List[torch.Tensor] = []
    qs: List[torch.Tensor] = []
    base = 0
    for _, dims in boxes:
        lz, ly, lx = dims
        ext = [L - abs(dd) for L, dd in zip(dims, d)]
        if min(ext) > 0:
            i = torch.arange(ext[0] * ext[1] * ext[2], device=dev, dtype=torch.int64)
            z = i // (ext[2] * ext[1]) + max(0, -d[0])
            y = (i // ext[2]) % ext[1] + max(0, -d[1])
            x = i % ext[2] + max(0, -d[2])
            q = base + (z * ly + y) * lx + x
            qs.append(q)
            ps.append(q + (d[0] * ly + d[1]) * lx + d[2])
        base += lz * ly * lx
    empty = torch.zeros(0, dtype=torch.int64, device=dev)
    return (torch.cat(ps) if ps else empty), (torch.cat(qs) if qs else empty)


def box_degree(boxes: Sequence[Box], K: int, dev) -> torch.Tensor:
    """Entries per output row (centre included), int64 [N]: per axis, the
    number of v + d (|d| <= r) inside [0, L), multiplied over the axes."""
    r = (K - 1) // 2
    parts = []
    for _, dims in boxes:
        lz, ly, lx = dims
        q = torch.arange(lz * ly * lx, device=dev, dtype=torch.int64)
        deg = torch.ones_like(q)
        for v, L in ((q // (lx * ly), lz), ((q // lx) % ly, ly), (q % lx, lx)):
            deg = deg * (torch.clamp(v + r, max=L - 1) - torch.clamp(v - r, min=0) + 1)
        parts.append(deg)
    return torch.cat(parts)
