"""TEST INFRASTRUCTURE ONLY — the oracle for submanifold sparse convolution.

Plain, slow CPU implementations of what the GPU path computes, used to judge
it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product library never does.  It
shares no code with the GPU path.

Contents
--------
``OracleMap`` / ``build_map`` / ``forward`` / ``forward_rows``
    ctypes front end of ``spconv_oracle.cpp`` (ordered-tree coordinate lookup,
    per-entry fp64 vector-matrix products).  See that file for the passages
    each step follows.
``build_map_strided`` / ``OracleMap.transpose``
    Strided maps (downsampling, regular output definition) and their
    transposes (upsampling); see ``spconv_oracle.cpp``.
``OracleMap.backward_data`` / ``OracleMap.backward_weights``
    The gradients of the forward with respect to its input features and its
    weights, each the chain rule of the forward's per-entry sum, in fp64.
``brute_map``
    O(N^2) pair test for tiny inputs: (j, q) is an entry of offset d iff
    coords[j] = coords[q] + (0, d).  Independent of the tree lookup.
``dense_grow``
    The regular ("dilating") output definition, for the dilation pins:
    "Sparse inputs and sparse convolution", section "What a dense convolution
    does to empty space", and the SparseConvNet blog, section 2 (regular
    output definition).
``adaptive_groups`` / ``padded_rows``
    The adaptive grouping of offsets into padded batched products (epsilon,
    S), from "TorchSparse: regular computation from irregular sparsity".
``mac_count``
    Entries x Cin x Cout: "Sparse inputs and sparse convolution", section
    "A symmetry you can check on the slide" (MACs per layer).

Every function here has a pin in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Dict, Iterable, List, Optional, Sequence, Set, Tuple

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None

STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "DUPLICATE_COORD", 3: "COORD_RANGE"}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status} ({STATUS_NAMES.get(status, '?')})")
        self.status = status
        self.name = STATUS_NAMES.get(status, "?")


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        # SPCONV_ORACLE_LIB names another build of the same source (the tests'
        # sanitizer build); by default the in-tree library, rebuilt when stale.
        path = os.environ.get("SPCONV_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_build_map.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
        lib.oracle_build_map.restype = ctypes.c_int
        lib.oracle_build_table.argtypes = lib.oracle_build_map.argtypes
        lib.oracle_build_table.restype = ctypes.c_int
        lib.oracle_map_free.argtypes = [ctypes.c_void_p]
        lib.oracle_map_free.restype = None
        lib.oracle_map_kernel.argtypes = [ctypes.c_void_p]
        lib.oracle_map_kernel.restype = ctypes.c_int32
        lib.oracle_map_count.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        lib.oracle_map_count.restype = ctypes.c_int64
        lib.oracle_map_list.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, _i32p]
        lib.oracle_map_list.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [ctypes.c_void_p, _f64p, _f64p, ctypes.c_int32, ctypes.c_int32, _f64p]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward_parallel.argtypes = lib.oracle_forward.argtypes + [ctypes.c_int32]
        lib.oracle_forward_parallel.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int32
        lib.oracle_backward_data.argtypes = lib.oracle_forward.argtypes
        lib.oracle_backward_data.restype = ctypes.c_int
        lib.oracle_backward_weights.argtypes = lib.oracle_forward.argtypes
        lib.oracle_backward_weights.restype = ctypes.c_int
        lib.oracle_backward_weights_parallel.argtypes = lib.oracle_forward.argtypes + [ctypes.c_int32]
        lib.oracle_backward_weights_parallel.restype = ctypes.c_int
        lib.oracle_forward_rows.argtypes = [ctypes.c_void_p, _f64p, _f64p, ctypes.c_int32, ctypes.c_int32,
                                            _i64p, ctypes.c_int64, _f64p]
        lib.oracle_forward_rows.restype = ctypes.c_int
        lib.oracle_neighbours.argtypes = [ctypes.c_void_p, _i64p, ctypes.c_int64, _i32p]
        lib.oracle_neighbours.restype = ctypes.c_int
        lib.oracle_build_map_strided.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_void_p)]
        lib.oracle_build_map_strided.restype = ctypes.c_int
        lib.oracle_transpose_map.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        lib.oracle_transpose_map.restype = ctypes.c_int
        lib.oracle_map_rows_in.argtypes = [ctypes.c_void_p]
        lib.oracle_map_rows_in.restype = ctypes.c_int64
        lib.oracle_map_rows_out.argtypes = [ctypes.c_void_p]
        lib.oracle_map_rows_out.restype = ctypes.c_int64
        lib.oracle_map_stride.argtypes = [ctypes.c_void_p]
        lib.oracle_map_stride.restype = ctypes.c_int32
        lib.oracle_map_out_coords.argtypes = [ctypes.c_void_p, _i32p]
        lib.oracle_map_out_coords.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class OracleMap:
    """Map built by the oracle.  ``lists[k]`` is ``(in_idx, out_idx)`` int32
    arrays ordered by output row.  With ``lists=False`` only the coordinate
    table is built: ``forward_rows`` and ``neighbours`` still work, the lists
    stay empty.  ``N`` is the number of input rows and ``N_out`` of output
    rows (equal for a submanifold map); strided and transposed maps (see
    ``build_map_strided``) also carry ``out_coords`` and ``stride``."""

    def __init__(self, coords: np.ndarray, K: int, lists: bool = True):
        coords = np.ascontiguousarray(np.asarray(coords, dtype=np.int32).reshape(-1, 4))
        h = ctypes.c_void_p()
        fn = _lib().oracle_build_map if lists else _lib().oracle_build_table
        st = fn(_ptr(coords, _i32p), int(coords.shape[0]), int(K), ctypes.byref(h))
        if st != 0:
            raise OracleError(st)
        self._load(h, K, coords, None, lists)

    @classmethod
    def _wrap(cls, h, K: int, coords: np.ndarray) -> "OracleMap":
        m = cls.__new__(cls)
        n_out = int(_lib().oracle_map_rows_out(h))
        out = np.empty((n_out, 4), np.int32)
        st = _lib().oracle_map_out_coords(h, _ptr(out, _i32p))
        if st != 0:
            _lib().oracle_map_free(h)
            raise OracleError(st)
        m._load(h, K, coords, out, True)
        return m

    def _load(self, h, K: int, coords: np.ndarray, out_coords: Optional[np.ndarray], lists: bool):
        self._h = h
        self.coords = coords
        self.K = int(K)
        self.N = int(_lib().oracle_map_rows_in(h))
        self.N_out = int(_lib().oracle_map_rows_out(h))
        self.stride = int(_lib().oracle_map_stride(h))
        self.out_coords = out_coords
        self.has_lists = bool(lists)
        kv = self.K ** 3
        self.counts = np.array([_lib().oracle_map_count(h, k) for k in range(kv)], dtype=np.int64)
        self.lists: List[Tuple[np.ndarray, np.ndarray]] = []
        for k in range(kv):
            a = np.empty(self.counts[k], np.int32)
            b = np.empty(self.counts[k], np.int32)
            if self.counts[k] > 0:
                st = _lib().oracle_map_list(h, k, _ptr(a, _i32p), _ptr(b, _i32p))
                if st != 0:
                    raise OracleError(st)
            self.lists.append((a, b))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.oracle_map_free(h)
            self._h = None

    @property
    def total_entries(self) -> int:
        return int(self.counts.sum())

    def forward(self, feats: np.ndarray, weights: np.ndarray) -> np.ndarray:
        """fp64 forward over the whole map (needs the lists).  ``feats`` [N, Cin] and ``weights``
        [K^3, Cin, Cout] are widened to fp64 exactly before the call."""
        if not self.has_lists:
            raise ValueError("built with lists=False: use forward_rows")
        f = np.ascontiguousarray(np.asarray(feats, dtype=np.float64))
        w = np.ascontiguousarray(np.asarray(weights, dtype=np.float64))
        cin, cout = w.shape[1], w.shape[2]
        assert f.shape == (self.N, cin) and w.shape[0] == self.K ** 3
        out = np.empty((self.N_out, cout), np.float64)
        st = _lib().oracle_forward(self._h, _ptr(f, _f64p), _ptr(w, _f64p), cin, cout, _ptr(out, _f64p))
        if st != 0:
            raise OracleError(st)
        return out

    def forward_parallel(self, feats: np.ndarray, weights: np.ndarray, threads: int = 0) -> np.ndarray:
        """The same fp64 forward split over output rows on ``threads`` OpenMP
        threads (0: all the runtime offers).  Same terms in the same order per
        output value as ``forward``, hence bit-identical to it."""
        if not self.has_lists:
            raise ValueError("built with lists=False: use forward_rows")
        f = np.ascontiguousarray(np.asarray(feats, dtype=np.float64))
        w = np.ascontiguousarray(np.asarray(weights, dtype=np.float64))
        cin, cout = w.shape[1], w.shape[2]
        assert f.shape == (self.N, cin) and w.shape[0] == self.K ** 3
        out = np.empty((self.N_out, cout), np.float64)
        st = _lib().oracle_forward_parallel(self._h, _ptr(f, _f64p), _ptr(w, _f64p), cin, cout,
                                            _ptr(out, _f64p), int(threads))
        if st != 0:
            raise OracleError(st)
        return out

    def transpose(self) -> "OracleMap":
        """The transposed map of a strided map (the upsampling convolution),
        built from its own definition: outputs are this map's inputs, inputs
        this map's outputs, entry (q, j) at offset d when s q + d = p_j."""
        h = ctypes.c_void_p()
        st = _lib().oracle_transpose_map(self._h, ctypes.byref(h))
        if st != 0:
            raise OracleError(st)
        return OracleMap._wrap(h, self.K, self.out_coords)

    def backward_data(self, grad_out: np.ndarray, weights: np.ndarray) -> np.ndarray:
        """fp64 gradient with respect to the input features: grad_in[j] = sum
        over entries (j, q) of offset k of grad_out[q] @ W[k]^T."""
        if not self.has_lists:
            raise ValueError("built with lists=False")
        g = np.ascontiguousarray(np.asarray(grad_out, dtype=np.float64))
        w = np.ascontiguousarray(np.asarray(weights, dtype=np.float64))
        cin, cout = w.shape[1], w.shape[2]
        assert g.shape == (self.N_out, cout) and w.shape[0] == self.K ** 3
        out = np.empty((self.N, cin), np.float64)
        st = _lib().oracle_backward_data(self._h, _ptr(g, _f64p), _ptr(w, _f64p), cin, cout, _ptr(out, _f64p))
        if st != 0:
            raise OracleError(st)
        return out

    def backward_weights(self, feats: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
        """fp64 gradient with respect to the weights: grad_w[k] = sum over
        entries (j, q) of offset k of the outer product feats[j] x grad_out[q]."""
        if not self.has_lists:
            raise ValueError("built with lists=False")
        f = np.ascontiguousarray(np.asarray(feats, dtype=np.float64))
        g = np.ascontiguousarray(np.asarray(grad_out, dtype=np.float64))
        cin, cout = f.shape[1], g.shape[1]
        assert f.shape[0] == self.N and g.shape[0] == self.N_out
        out = np.empty((self.K ** 3, cin, cout), np.float64)
        st = _lib().oracle_backward_weights(self._h, _ptr(f, _f64p), _ptr(g, _f64p), cin, cout, _ptr(out, _f64p))
        if st != 0:
            raise OracleError(st)
        return out

    def backward_weights_parallel(self, feats: np.ndarray, grad_out: np.ndarray, threads: int = 0) -> np.ndarray:
        """``backward_weights`` with the offsets split over OpenMP threads
        (same terms in the same order per value: bit-identical)."""
        if not self.has_lists:
            raise ValueError("built with lists=False")
        f = np.ascontiguousarray(np.asarray(feats, dtype=np.float64))
        g = np.ascontiguousarray(np.asarray(grad_out, dtype=np.float64))
        cin, cout = f.shape[1], g.shape[1]
        assert f.shape[0] == self.N and g.shape[0] == self.N_out
        out = np.empty((self.K ** 3, cin, cout), np.float64)
        st = _lib().oracle_backward_weights_parallel(self._h, _ptr(f, _f64p), _ptr(g, _f64p), cin, cout,
                                                     _ptr(out, _f64p), int(threads))
        if st != 0:
            raise OracleError(st)
        return out

    def forward_rows(self, feats: np.ndarray, weights: np.ndarray, rows: Sequence[int]) -> np.ndarray:
        """fp64 forward for selected output rows, evaluated from the coordinate
        table one row at a time."""
        f = np.ascontiguousarray(np.asarray(feats, dtype=np.float64))
        w = np.ascontiguousarray(np.asarray(weights, dtype=np.float64))
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        cin, cout = w.shape[1], w.shape[2]
        out = np.empty((r.shape[0], cout), np.float64)
        st = _lib().oracle_forward_rows(self._h, _ptr(f, _f64p), _ptr(w, _f64p), cin, cout,
                                        _ptr(r, _i64p), r.shape[0], _ptr(out, _f64p))
        if st != 0:
            raise OracleError(st)
        return out

    def neighbours(self, rows: Sequence[int]) -> np.ndarray:
        """[len(rows), K^3] neighbour rows (or -1) of selected outputs."""
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nbr = np.empty((r.shape[0], self.K ** 3), np.int32)
        st = _lib().oracle_neighbours(self._h, _ptr(r, _i64p), r.shape[0], _ptr(nbr, _i32p))
        if st != 0:
            raise OracleError(st)
        return nbr


def build_map(coords: np.ndarray, K: int) -> OracleMap:
    return OracleMap(coords, K)


def build_map_strided(coords: np.ndarray, K: int, stride: int) -> OracleMap:
    """Map of a strided convolution with a K^3 kernel (offset components
    -floor((K-1)/2) .. +K-1-floor((K-1)/2)) and stride ``stride``, outputs by
    the regular output definition in lexicographic (b, z, y, x) order (see
    ``oracle_build_map_strided``)."""
    coords = np.ascontiguousarray(np.asarray(coords, dtype=np.int32).reshape(-1, 4))
    h = ctypes.c_void_p()
    st = _lib().oracle_build_map_strided(_ptr(coords, _i32p), int(coords.shape[0]), int(K), int(stride),
                                         ctypes.byref(h))
    if st != 0:
        raise OracleError(st)
    return OracleMap._wrap(h, K, coords)


def offset_of_any(k: int, K: int) -> Tuple[int, int, int]:
    """Offset of index k for any kernel size: components lo .. lo + K - 1,
    lo = -floor((K - 1) / 2) (odd K: the centred offsets of ``offset_of``)."""
    lo = -((K - 1) // 2)
    return (k // (K * K) + lo, (k // K) % K + lo, k % K + lo)


def build_table(coords: np.ndarray, K: int) -> OracleMap:
    """Coordinate table only, for row-at-a-time evaluation."""
    return OracleMap(coords, K, lists=False)


def max_threads() -> int:
    """Threads the oracle's parallel forward uses by default."""
    return int(_lib().oracle_max_threads())


def offset_index(dz: int, dy: int, dx: int, K: int) -> int:
    """k(d) = ((dz + r) K + (dy + r)) K + (dx + r), r = (K - 1) / 2."""
    r = (K - 1) // 2
    return ((dz + r) * K + (dy + r)) * K + (dx + r)


def offset_of(k: int, K: int) -> Tuple[int, int, int]:
    r = (K - 1) // 2
    return (k // (K * K) - r, (k // K) % K - r, k % K - r)


def brute_map(coords: np.ndarray, K: int) -> Dict[int, Set[Tuple[int, int]]]:
    """Per-offset entry sets by an O(N^2) pair test: (j, q) belongs to offset
    d = coords[j] - coords[q] when both share b and max |d| <= r.  For tiny
    inputs only."""
    c = np.asarray(coords, dtype=np.int64).reshape(-1, 4)
    r = (K - 1) // 2
    res: Dict[int, Set[Tuple[int, int]]] = {k: set() for k in range(K ** 3)}
    for q in range(c.shape[0]):
        d = c - c[q]
        ok = (d[:, 0] == 0) & (np.abs(d[:, 1:]).max(axis=1) <= r)
        for j in np.nonzero(ok)[0]:
            dz, dy, dx = (int(v) for v in d[j, 1:])
            res[offset_index(dz, dy, dx, K)].add((int(j), int(q)))
    return res


def dense_grow(active: Iterable[Tuple[int, ...]], layers: int, shape: Optional[Tuple[int, ...]] = None,
               K: int = 3) -> Set[Tuple[int, ...]]:
    """Active sites after ``layers`` dense K^d convolutions under the regular
    output definition: an output is active when its window touches any active
    input.  ``shape`` clips to a grid (the slide grid); None means unbounded."""
    cur = set(tuple(int(v) for v in a) for a in active)
    if not cur:
        return cur
    d = len(next(iter(cur)))
    r = (K - 1) // 2
    offs = list(itertools.product(range(-r, r + 1), repeat=d))
    for _ in range(layers):
        nxt = set()
        for a in cur:
            for o in offs:
                p = tuple(a[i] + o[i] for i in range(d))
                if shape is None or all(0 <= p[i] < shape[i] for i in range(d)):
                    nxt.add(p)
        cur = nxt
    return cur


def conventional_entries(active: Iterable[Tuple[int, ...]], shape: Tuple[int, ...], K: int = 3) -> int:
    """Entries of a conventional (zero-skipping) layer: one per active input
    and in-grid output position its window reaches."""
    act = [tuple(int(v) for v in a) for a in active]
    d = len(act[0])
    r = (K - 1) // 2
    n = 0
    for a in act:
        for o in itertools.product(range(-r, r + 1), repeat=d):
            if all(0 <= a[i] + o[i] < shape[i] for i in range(d)):
                n += 1
    return n


def adaptive_groups(counts: Sequence[int], epsilon: float, S: float, centre: Optional[int] = None) -> List[List[int]]:
    """Offset groups of the adaptive grouping of "TorchSparse: regular
    computation from irregular sparsity", sections "The spectrum: separate,
    dense, grouped" and "How the groups are chosen".

    The offsets with entries, the identity offset ``centre`` apart (it runs
    on its own), are walked in decreasing map size (ties by index) and cut
    into runs: a run grows while its redundant computation ratio, the padded
    rows over all rows of the padded batch (m x max - sum) / (m x max), stays
    at or below ``epsilon``, and a new run starts the moment the next offset
    would take it above.  A run whose largest map is at least ``S`` runs as
    separate matrix products (each offset its own group); the others run as
    one batched product each, padded to their largest map.  So epsilon = 1
    with S unbounded is one dense batch, S = 0 is separate computation, and
    epsilon = 0 groups offsets of equal map size only (the mirror pairs of a
    submanifold map: symmetric grouping).  The centre, when given and
    non-empty, comes first as a group of its own.

    The page describes the paper's two-pointer scan in kernel order but sorts
    by map size in its worked figure and its tuner; the size order is the one
    under which epsilon = 0 is the symmetric grouping it names (the mirror
    offsets k and K^3 - 1 - k are never adjacent in kernel order), so it is
    the order taken here."""
    order = sorted((k for k in range(len(counts)) if counts[k] > 0 and k != centre),
                   key=lambda k: (-int(counts[k]), k))
    runs: List[List[int]] = []
    cur: List[int] = []
    for k in order:
        cand = cur + [k]
        mx = max(int(counts[j]) for j in cand)
        tot = sum(int(counts[j]) for j in cand)
        ratio = (len(cand) * mx - tot) / (len(cand) * mx)
        if cur and ratio > epsilon:
            runs.append(cur)
            cur = [k]
        else:
            cur = cand
    if cur:
        runs.append(cur)
    groups: List[List[int]] = []
    if centre is not None and counts[centre] > 0:
        groups.append([centre])
    for g in runs:
        if max(int(counts[j]) for j in g) >= S:
            groups.extend([[j] for j in g])
        else:
            groups.append(g)
    return groups


def padded_rows(counts: Sequence[int], groups: Sequence[Sequence[int]]) -> int:
    """Rows the grouped computation runs: every member of a group padded to
    the group's largest map."""
    return sum(len(g) * max(int(counts[j]) for j in g) for g in groups)


def mac_count(entries: int, cin: int, cout: int) -> int:
    """Multiply-accumulates of a layer: entries x Cin x Cout, independent of
    how the entries are grouped."""
    return int(entries) * int(cin) * int(cout)
