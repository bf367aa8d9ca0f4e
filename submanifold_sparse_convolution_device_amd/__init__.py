"""Submanifold sparse convolution on AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libspconv.so`` (declared in
``include/spconv.h``).  It only marshals arguments: PyTorch tensors supply
device memory and the current HIP stream; every step of the map build and the
forward runs in the library's HIP kernels.  There is no CPU fallback: if the
library is missing, every entry point raises.

The raw C functions are exposed under their C names (``spconv_build_map``,
``spconv_forward``, ...) through :func:`lib`; :func:`build_map` and
:func:`forward` wrap them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPCONV_LIB_PATH names another build of the same library (the tests' host-only
# sanitizer build); by default the in-tree libspconv.so.
LIB_PATH = os.environ.get("SPCONV_LIB_PATH") or os.path.join(_HERE, "libspconv.so")

STATUS = {
    0: "SPCONV_OK",
    1: "SPCONV_ERR_INVALID_ARG",
    2: "SPCONV_ERR_DUPLICATE_COORD",
    3: "SPCONV_ERR_COORD_RANGE",
    4: "SPCONV_ERR_UNSUPPORTED",
    5: "SPCONV_ERR_OUT_OF_MEMORY",
    6: "SPCONV_ERR_DEVICE",
}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

# Every symbol include/spconv.h declares.
EXPORTED = (
    "spconv_abi_version", "spconv_build_map", "spconv_build_map_async", "spconv_map_wait",
    "spconv_map_info", "spconv_map_counts", "spconv_map_lists", "spconv_forward",
    "spconv_forward_noalloc", "spconv_backward_data", "spconv_backward_weights", "spconv_build_map_strided",
    "spconv_map_transpose", "spconv_map_geometry", "spconv_map_out_coords", "spconv_group_plan", "spconv_group_plan_counts",
    "spconv_forward_grouped", "spconv_select_dataflow", "spconv_map_free", "spconv_status_string",
    "spconv_last_error", "spconv_weights_prepare", "spconv_forward_prepared", "spconv_weights_free",
)
MAP_KINDS = {0: "submanifold", 1: "strided", 2: "transposed"}
DATAFLOWS = {0: "fused", 1: "grouped"}


class spconv_dataflow(ctypes.Structure):
    """Mirror of the C struct spconv_dataflow."""
    _fields_ = [("kind", ctypes.c_int32), ("groups", ctypes.c_int32), ("epsilon", ctypes.c_double),
                ("S", ctypes.c_double), ("ms", ctypes.c_float), ("fused_ms", ctypes.c_float),
                ("candidates", ctypes.c_int32), ("reserved", ctypes.c_int32)]

_LIB: Optional[ctypes.CDLL] = None


class SpconvError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.name}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded ``libspconv.so`` with argument types declared."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc for gfx950) first")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes the library bind to that one runtime, so
    # torch's stream handles and allocations are valid in both.
    _torch()
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _mapped_hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped in this process: {runtimes}")
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.spconv_abi_version.argtypes, L.spconv_abi_version.restype = [], i32
    L.spconv_build_map.argtypes = [vp, i64, i32, vp, ctypes.POINTER(vp)]
    L.spconv_build_map.restype = ctypes.c_int
    L.spconv_build_map_async.argtypes = [vp, i64, i32, vp, ctypes.POINTER(vp)]
    L.spconv_build_map_async.restype = ctypes.c_int
    L.spconv_map_wait.argtypes, L.spconv_map_wait.restype = [vp], ctypes.c_int
    L.spconv_map_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.spconv_map_info.restype = ctypes.c_int
    L.spconv_map_counts.argtypes = [vp, vp, vp]
    L.spconv_map_counts.restype = ctypes.c_int
    L.spconv_map_lists.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    L.spconv_map_lists.restype = ctypes.c_int
    L.spconv_forward.argtypes = [vp, vp, vp, i32, i32, ctypes.c_int, vp, vp]
    L.spconv_forward.restype = ctypes.c_int
    L.spconv_forward_noalloc.argtypes = L.spconv_forward.argtypes
    L.spconv_forward_noalloc.restype = ctypes.c_int
    L.spconv_weights_prepare.argtypes = [vp, i32, i32, i32, ctypes.c_int, vp, ctypes.POINTER(vp)]
    L.spconv_weights_prepare.restype = ctypes.c_int
    L.spconv_forward_prepared.argtypes = [vp, vp, vp, vp, vp]
    L.spconv_forward_prepared.restype = ctypes.c_int
    L.spconv_weights_free.argtypes, L.spconv_weights_free.restype = [vp], None
    L.spconv_backward_data.argtypes = L.spconv_forward.argtypes
    L.spconv_backward_data.restype = ctypes.c_int
    L.spconv_backward_weights.argtypes = L.spconv_forward.argtypes
    L.spconv_backward_weights.restype = ctypes.c_int
    L.spconv_build_map_strided.argtypes = [vp, i64, i32, i32, vp, ctypes.POINTER(vp)]
    L.spconv_build_map_strided.restype = ctypes.c_int
    L.spconv_map_transpose.argtypes = [vp, vp, ctypes.POINTER(vp)]
    L.spconv_map_transpose.restype = ctypes.c_int
    L.spconv_map_geometry.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i32),
                                      ctypes.POINTER(i32)]
    L.spconv_map_geometry.restype = ctypes.c_int
    L.spconv_map_out_coords.argtypes = [vp, ctypes.POINTER(vp)]
    L.spconv_map_out_coords.restype = ctypes.c_int
    f64, pi32 = ctypes.c_double, ctypes.POINTER(i32)
    L.spconv_group_plan.argtypes = [vp, f64, f64, i32, pi32, pi32, pi32, pi32, ctypes.POINTER(i64)]
    L.spconv_group_plan.restype = ctypes.c_int
    L.spconv_group_plan_counts.argtypes = [ctypes.POINTER(i64), i32, i32, f64, f64, i32, pi32, pi32, pi32, pi32,
                                           ctypes.POINTER(i64)]
    L.spconv_group_plan_counts.restype = ctypes.c_int
    L.spconv_forward_grouped.argtypes = [vp, vp, vp, i32, i32, ctypes.c_int, f64, f64, vp, vp]
    L.spconv_forward_grouped.restype = ctypes.c_int
    L.spconv_select_dataflow.argtypes = [vp, vp, vp, i32, i32, ctypes.c_int, ctypes.POINTER(f64), i32,
                                         ctypes.POINTER(f64), i32, i32, vp, vp, ctypes.POINTER(spconv_dataflow)]
    L.spconv_select_dataflow.restype = ctypes.c_int
    L.spconv_map_free.argtypes, L.spconv_map_free.restype = [vp], None
    L.spconv_status_string.argtypes, L.spconv_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.spconv_last_error.argtypes, L.spconv_last_error.restype = [], ctypes.c_char_p
    # the runtime's own copy routine, resolved through the library's dependencies
    L.hipMemcpyAsync.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    L.hipMemcpyAsync.restype = ctypes.c_int
    _LIB = L
    return L


def _mapped_hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({l.split()[-1] for l in f if "libamdhip64" in l})
    except OSError:
        return []


def _check(status: int) -> None:
    if status != 0:
        raise SpconvError(status, lib().spconv_last_error().decode(errors="replace"))


# ------------------------------------------------------------------ raw C names


def spconv_abi_version() -> int:
    return int(lib().spconv_abi_version())


def spconv_build_map(d_coords: int, n: int, kernel_size: int, hip_stream: int) -> int:
    """Raw call: returns the map handle (int) or raises SpconvError."""
    h = ctypes.c_void_p()
    _check(lib().spconv_build_map(d_coords, n, kernel_size, hip_stream, ctypes.byref(h)))
    return int(h.value)


def spconv_build_map_async(d_coords: int, n: int, kernel_size: int, hip_stream: int) -> int:
    """Raw call: enqueues the build and returns the map handle (int); device
    errors surface in spconv_map_wait / spconv_map_info / spconv_map_counts."""
    h = ctypes.c_void_p()
    _check(lib().spconv_build_map_async(d_coords, n, kernel_size, hip_stream, ctypes.byref(h)))
    return int(h.value)


def spconv_map_wait(handle: int) -> None:
    _check(lib().spconv_map_wait(handle))


def spconv_map_info(handle: int) -> Tuple[int, int, int]:
    K, n, e = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().spconv_map_info(handle, ctypes.byref(K), ctypes.byref(n), ctypes.byref(e)))
    return K.value, n.value, e.value


def spconv_map_counts(handle: int, kernel_volume: int) -> Tuple[np.ndarray, np.ndarray]:
    counts = np.zeros(kernel_volume, np.int64)
    offsets = np.zeros(kernel_volume + 1, np.int64)
    _check(lib().spconv_map_counts(handle, counts.ctypes.data, offsets.ctypes.data))
    return counts, offsets


def spconv_map_lists(handle: int) -> Tuple[int, int]:
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().spconv_map_lists(handle, ctypes.byref(a), ctypes.byref(b)))
    return int(a.value or 0), int(b.value or 0)


def spconv_forward(d_feats: int, d_weights: int, handle: int, c_in: int, c_out: int, dtype: int,
                   d_out: int, hip_stream: int) -> None:
    _check(lib().spconv_forward(d_feats, d_weights, handle, c_in, c_out, dtype, d_out, hip_stream))


def spconv_forward_noalloc(d_feats: int, d_weights: int, handle: int, c_in: int, c_out: int, dtype: int,
                           d_out: int, hip_stream: int) -> None:
    _check(lib().spconv_forward_noalloc(d_feats, d_weights, handle, c_in, c_out, dtype, d_out, hip_stream))


def spconv_weights_prepare(d_weights: int, kernel_volume: int, c_in: int, c_out: int, dtype: int,
                           hip_stream: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().spconv_weights_prepare(d_weights, kernel_volume, c_in, c_out, dtype, hip_stream, ctypes.byref(h)))
    return int(h.value)


def spconv_forward_prepared(d_feats: int, weights: int, handle: int, d_out: int, hip_stream: int) -> None:
    _check(lib().spconv_forward_prepared(d_feats, weights, handle, d_out, hip_stream))


def spconv_weights_free(weights: int) -> None:
    lib().spconv_weights_free(weights)


def spconv_backward_data(d_grad_out: int, d_weights: int, handle: int, c_in: int, c_out: int, dtype: int,
                         d_grad_in: int, hip_stream: int) -> None:
    _check(lib().spconv_backward_data(d_grad_out, d_weights, handle, c_in, c_out, dtype, d_grad_in, hip_stream))


def spconv_backward_weights(d_feats: int, d_grad_out: int, handle: int, c_in: int, c_out: int, dtype: int,
                            d_grad_w: int, hip_stream: int) -> None:
    _check(lib().spconv_backward_weights(d_feats, d_grad_out, handle, c_in, c_out, dtype, d_grad_w, hip_stream))


def spconv_build_map_strided(d_coords: int, n_in: int, kernel_size: int, stride: int, hip_stream: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().spconv_build_map_strided(d_coords, n_in, kernel_size, stride, hip_stream, ctypes.byref(h)))
    return int(h.value)


def spconv_map_transpose(handle: int, hip_stream: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().spconv_map_transpose(handle, hip_stream, ctypes.byref(h)))
    return int(h.value)


def spconv_map_geometry(handle: int) -> Tuple[int, int, int, int]:
    n_in, n_out = ctypes.c_int64(), ctypes.c_int64()
    stride, kind = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().spconv_map_geometry(handle, ctypes.byref(n_in), ctypes.byref(n_out), ctypes.byref(stride),
                                     ctypes.byref(kind)))
    return n_in.value, n_out.value, stride.value, kind.value


def spconv_map_out_coords(handle: int) -> int:
    p = ctypes.c_void_p()
    _check(lib().spconv_map_out_coords(handle, ctypes.byref(p)))
    return int(p.value or 0)


def spconv_group_plan(handle: int, epsilon: float, S: float, kernel_volume: int):
    """(offsets, groups, n_groups, padded_rows) of the plan: offsets and
    group indices of the entries in execution order."""
    offs = (ctypes.c_int32 * kernel_volume)()
    grp = (ctypes.c_int32 * kernel_volume)()
    n, ng, pad = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().spconv_group_plan(handle, float(epsilon), float(S), kernel_volume, offs, grp, ctypes.byref(n),
                                   ctypes.byref(ng), ctypes.byref(pad)))
    return list(offs[:n.value]), list(grp[:n.value]), ng.value, pad.value


def spconv_group_plan_counts(counts, epsilon: float, S: float, centre: int = -1):
    """(offsets, groups, n_groups, padded_rows) of the plan over the given
    per-offset map sizes (no map, no device)."""
    kv = len(counts)
    arr = (ctypes.c_int64 * max(kv, 1))(*[int(c) for c in counts])
    offs = (ctypes.c_int32 * max(kv, 1))()
    grp = (ctypes.c_int32 * max(kv, 1))()
    n, ng, pad = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().spconv_group_plan_counts(arr, kv, int(centre), float(epsilon), float(S), kv, offs, grp,
                                          ctypes.byref(n), ctypes.byref(ng), ctypes.byref(pad)))
    return list(offs[:n.value]), list(grp[:n.value]), ng.value, pad.value


def spconv_forward_grouped(d_feats: int, d_weights: int, handle: int, c_in: int, c_out: int, dtype: int,
                           epsilon: float, S: float, d_out: int, hip_stream: int) -> None:
    _check(lib().spconv_forward_grouped(d_feats, d_weights, handle, c_in, c_out, dtype, float(epsilon), float(S),
                                        d_out, hip_stream))


def spconv_select_dataflow(d_feats: int, d_weights: int, handle: int, c_in: int, c_out: int, dtype: int,
                           epsilons, thresholds, reps: int, d_out: int, hip_stream: int) -> spconv_dataflow:
    def grid(v):
        if v is None:
            return None, 0
        arr = (ctypes.c_double * len(v))(*[float(x) for x in v])
        return arr, len(v)
    e, ne = grid(epsilons)
    t, nt = grid(thresholds)
    best = spconv_dataflow()
    _check(lib().spconv_select_dataflow(d_feats, d_weights, handle, c_in, c_out, dtype, e, ne, t, nt, int(reps),
                                        d_out, hip_stream, ctypes.byref(best)))
    return best


def spconv_map_free(handle: int) -> None:
    lib().spconv_map_free(handle)


def spconv_status_string(status: int) -> str:
    return lib().spconv_status_string(status).decode()


def spconv_last_error() -> str:
    return lib().spconv_last_error().decode(errors="replace")


# ------------------------------------------------------------------ torch front end


def _torch():
    import torch
    return torch


def _stream() -> int:
    """Handle of torch's current stream on the current device."""
    return int(_torch().cuda.current_stream().cuda_stream)


class _OnDevice:
    """Makes ``device`` current for the call only when it is not already."""

    __slots__ = ("idx", "prev")

    def __init__(self, device):
        self.idx = device.index if device.index is not None else 0
        self.prev = None

    def __enter__(self):
        torch = _torch()
        cur = torch.cuda.current_device()
        if cur != self.idx:
            self.prev = cur
            torch.cuda.set_device(self.idx)

    def __exit__(self, *exc):
        if self.prev is not None:
            _torch().cuda.set_device(self.prev)


class SpconvMap:
    """A kernel map on the GPU (owns the C handle).  ``n`` is its number of
    output rows and ``n_in`` of input rows (equal for a submanifold map);
    ``kind`` is "submanifold", "strided" or "transposed"."""

    def __init__(self, handle: int, device, kernel_size: int, n: int, n_in: Optional[int] = None,
                 stride: int = 1, kind: str = "submanifold"):
        self.handle = handle
        self.device = device
        self.kernel_size, self.n = kernel_size, n
        self.n_in = n if n_in is None else n_in
        self.stride, self.kind = stride, kind
        self.kernel_volume = self.kernel_size ** 3
        self._counts = None
        self._total = None

    @classmethod
    def _from_handle(cls, h: int, device, kernel_size: int) -> "SpconvMap":
        n_in, n_out, stride, kind = spconv_map_geometry(h)
        return cls(h, device, kernel_size, n_out, n_in, stride, MAP_KINDS[kind])

    def out_coords(self):
        """Output coordinates (int32 [n, 4] device tensor, a stream-ordered
        copy) of a strided or transposed map."""
        torch = _torch()
        src = spconv_map_out_coords(self.handle)
        out = torch.empty((self.n, 4), dtype=torch.int32, device=self.device)
        if self.n:
            with _OnDevice(self.device):
                rc = lib().hipMemcpyAsync(out.data_ptr(), src, 16 * self.n, 3, _stream())
                if rc != 0:
                    raise SpconvError(6, f"hipMemcpyAsync failed with {rc}")
        return out

    def transpose(self) -> "SpconvMap":
        """The transposed (upsampling) map of a strided map."""
        with _OnDevice(self.device):
            h = spconv_map_transpose(self.handle, _stream())
        return SpconvMap._from_handle(h, self.device, self.kernel_size)

    def wait(self) -> None:
        """Waits for the build (a no-op once done); raises its device error."""
        spconv_map_wait(self.handle)

    @property
    def total_entries(self) -> int:
        if self._total is None:
            self._total = spconv_map_info(self.handle)[2]
        return self._total

    def _load_counts(self):
        if self._counts is None:
            self._counts = spconv_map_counts(self.handle, self.kernel_volume)
        return self._counts

    @property
    def counts(self) -> np.ndarray:
        """Entries per offset, int64 [K^3]."""
        return self._load_counts()[0]

    @property
    def offsets(self) -> np.ndarray:
        """List offsets, int64 [K^3 + 1]."""
        return self._load_counts()[1]

    def lists(self):
        """(in_idx, out_idx) as int32 device tensors: stream-ordered copies of
        the map's lists (the map owns the originals)."""
        torch = _torch()
        a, b = spconv_map_lists(self.handle)
        e = self.total_entries
        out = torch.empty((2, e), dtype=torch.int32, device=self.device)
        if e:
            with _OnDevice(self.device):
                stream = _stream()
                for dst, src in ((out[0].data_ptr(), a), (out[1].data_ptr(), b)):
                    rc = lib().hipMemcpyAsync(dst, src, 4 * e, 3, stream)  # device to device
                    if rc != 0:
                        raise SpconvError(6, f"hipMemcpyAsync failed with {rc}")
        return out[0], out[1]

    def free(self):
        if self.handle:
            spconv_map_free(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def build_map(coords, kernel_size: int, wait: bool = True) -> SpconvMap:
    """Kernel map of a K^3 submanifold convolution over int32 [N, 4]
    (b, z, y, x) coordinates resident on a HIP device.  With wait=False the
    build is only enqueued (device errors then surface in ``SpconvMap.wait``
    or the first query of counts)."""
    torch = _torch()
    if not (isinstance(coords, torch.Tensor) and coords.is_cuda and coords.dtype == torch.int32
            and coords.dim() == 2 and coords.shape[1] == 4 and coords.is_contiguous()):
        raise SpconvError(1, "coords must be a contiguous int32 [N, 4] tensor on a HIP device")
    call = spconv_build_map if wait else spconv_build_map_async
    with _OnDevice(coords.device):
        h = call(coords.data_ptr(), coords.shape[0], int(kernel_size), _stream())
    return SpconvMap(h, coords.device, int(kernel_size), int(coords.shape[0]))


def build_map_strided(coords, kernel_size: int, stride: int) -> SpconvMap:
    """Kernel map of a strided (downsampling) convolution with a K^3 kernel
    (offset components -floor((K-1)/2) ..) over int32 [N, 4] coordinates on a
    HIP device; its outputs (``out_coords``) follow the regular output
    definition in lexicographic order."""
    torch = _torch()
    if not (isinstance(coords, torch.Tensor) and coords.is_cuda and coords.dtype == torch.int32
            and coords.dim() == 2 and coords.shape[1] == 4 and coords.is_contiguous()):
        raise SpconvError(1, "coords must be a contiguous int32 [N, 4] tensor on a HIP device")
    with _OnDevice(coords.device):
        h = spconv_build_map_strided(coords.data_ptr(), coords.shape[0], int(kernel_size), int(stride), _stream())
    return SpconvMap._from_handle(h, coords.device, int(kernel_size))


_DT = None


def forward(feats, weights, kmap: SpconvMap, out=None, noalloc=False):
    """f_out = sparse convolution of feats [n_in, C_in] with weights
    [K^3, C_in, C_out] over ``kmap``; returns out [n, C_out] (same dtype;
    n_in = n for a submanifold map).
    With ``noalloc`` the call goes to ``spconv_forward_noalloc`` (the
    library's fixed per-device scratch instead of an allocated workspace;
    ``out`` must then be given, so that nothing is allocated here either)."""
    global _DT
    torch = _torch()
    if _DT is None:
        _DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if not (feats.is_cuda and weights.is_cuda and feats.is_contiguous() and weights.is_contiguous()):
        raise SpconvError(1, "feats and weights must be contiguous tensors on a HIP device")
    if feats.dim() != 2 or weights.dim() != 3:
        raise SpconvError(1, "feats must be [N, C_in] and weights [K^3, C_in, C_out]")
    n_in, cin = feats.shape
    n = kmap.n
    kv, wcin, cout = weights.shape
    if n_in != kmap.n_in or kv != kmap.kernel_volume or wcin != cin:
        raise SpconvError(1, f"shape mismatch: feats {tuple(feats.shape)}, weights "
                             f"{tuple(weights.shape)}, map n_in={kmap.n_in} K^3={kmap.kernel_volume}")
    dt = feats.dtype
    if weights.dtype != dt:
        raise SpconvError(1, "feats and weights must share one dtype")
    code = _DT.get(dt)
    if code is None:
        raise SpconvError(4, f"dtype {dt} not supported")
    if out is None:
        if noalloc:
            raise SpconvError(1, "noalloc needs a caller-allocated out")
        out = torch.empty((n, cout), dtype=dt, device=feats.device)
    elif not (out.is_cuda and out.is_contiguous() and out.dtype == dt and tuple(out.shape) == (n, cout)):
        raise SpconvError(1, "out must be a contiguous [N, C_out] tensor of the feature dtype")
    with _OnDevice(feats.device):
        fn = spconv_forward_noalloc if noalloc else spconv_forward
        fn(feats.data_ptr(), weights.data_ptr(), kmap.handle, cin, cout, code, out.data_ptr(), _stream())
    return out


class PreparedWeights:
    """A layer's weights copied once for repeated forwards
    (``spconv_weights_prepare``); later changes to the tensor it was made
    from do not reach it."""

    def __init__(self, weights):
        global _DT
        torch = _torch()
        if _DT is None:
            _DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
        if not (weights.is_cuda and weights.is_contiguous() and weights.dim() == 3):
            raise SpconvError(1, "weights must be a contiguous [K^3, C_in, C_out] tensor on a HIP device")
        code = _DT.get(weights.dtype)
        if code is None:
            raise SpconvError(4, f"dtype {weights.dtype} not supported")
        self.kernel_volume, self.c_in, self.c_out = (int(v) for v in weights.shape)
        self.dtype, self.device, self.handle = weights.dtype, weights.device, None
        with _OnDevice(weights.device):
            self.handle = spconv_weights_prepare(weights.data_ptr(), self.kernel_volume, self.c_in, self.c_out,
                                                 code, _stream())

    def free(self) -> None:
        if self.handle:
            spconv_weights_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def prepare_weights(weights) -> PreparedWeights:
    """Prepares [K^3, C_in, C_out] weights for ``forward_prepared``."""
    return PreparedWeights(weights)


def forward_prepared(feats, pw: PreparedWeights, kmap: SpconvMap, out=None):
    """``forward`` with prepared weights (bit-identical output)."""
    torch = _torch()
    if pw.handle is None:
        raise SpconvError(1, "the prepared weights were freed")
    if not (feats.is_cuda and feats.is_contiguous() and feats.dim() == 2 and feats.dtype == pw.dtype):
        raise SpconvError(1, "feats must be a contiguous [N, C_in] tensor on a HIP device of the weights' dtype")
    if feats.shape[0] != kmap.n_in or feats.shape[1] != pw.c_in or pw.kernel_volume != kmap.kernel_volume:
        raise SpconvError(1, f"shape mismatch: feats {tuple(feats.shape)}, weights "
                             f"[{pw.kernel_volume}, {pw.c_in}, {pw.c_out}], map n_in={kmap.n_in} "
                             f"K^3={kmap.kernel_volume}")
    if out is None:
        out = torch.empty((kmap.n, pw.c_out), dtype=pw.dtype, device=feats.device)
    elif not (out.is_cuda and out.is_contiguous() and out.dtype == pw.dtype and tuple(out.shape) == (kmap.n, pw.c_out)):
        raise SpconvError(1, "out must be a contiguous [N, C_out] tensor of the feature dtype")
    with _OnDevice(feats.device):
        spconv_forward_prepared(feats.data_ptr(), pw.handle, kmap.handle, out.data_ptr(), _stream())
    return out


def _check_pair(a, b, kmap: SpconvMap, what, rows_a=None):
    rows_a = kmap.n if rows_a is None else rows_a
    if not (a.is_cuda and b.is_cuda and a.is_contiguous() and b.is_contiguous()):
        raise SpconvError(1, f"{what} must be contiguous tensors on a HIP device")
    if a.dim() != 2 or b.dim() != 2 or a.shape[0] != rows_a or b.shape[0] != kmap.n:
        raise SpconvError(1, f"{what} must be [{rows_a}, C] and [{kmap.n}, C]")
    if a.dtype != b.dtype:
        raise SpconvError(1, f"{what} must share one dtype")


def backward_data(grad_out, weights, kmap: SpconvMap, out=None):
    """Gradient of ``forward`` with respect to its features: grad_in
    [N, C_in] from grad_out [N, C_out] and the forward's weights
    [K^3, C_in, C_out] (same dtype)."""
    global _DT
    torch = _torch()
    if _DT is None:
        _DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if not (weights.is_cuda and weights.is_contiguous() and weights.dim() == 3):
        raise SpconvError(1, "weights must be a contiguous [K^3, C_in, C_out] tensor on a HIP device")
    kv, cin, cout = weights.shape
    _check_pair(grad_out, grad_out, kmap, "grad_out")
    if kv != kmap.kernel_volume or grad_out.shape[1] != cout or weights.dtype != grad_out.dtype:
        raise SpconvError(1, f"shape mismatch: grad_out {tuple(grad_out.shape)}, weights {tuple(weights.shape)}")
    code = _DT.get(grad_out.dtype)
    if code is None:
        raise SpconvError(4, f"dtype {grad_out.dtype} not supported")
    if out is None:
        out = torch.empty((kmap.n_in, cin), dtype=grad_out.dtype, device=grad_out.device)
    elif not (out.is_cuda and out.is_contiguous() and out.dtype == grad_out.dtype
              and tuple(out.shape) == (kmap.n_in, cin)):
        raise SpconvError(1, "out must be a contiguous [n_in, C_in] tensor of the gradient dtype")
    with _OnDevice(grad_out.device):
        spconv_backward_data(grad_out.data_ptr(), weights.data_ptr(), kmap.handle, cin, cout, code, out.data_ptr(),
                             _stream())
    return out


def backward_weights(feats, grad_out, kmap: SpconvMap, out=None):
    """Gradient of ``forward`` with respect to its weights: fp32
    [K^3, C_in, C_out] from feats [n_in, C_in] and grad_out [n, C_out]."""
    global _DT
    torch = _torch()
    if _DT is None:
        _DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    _check_pair(feats, grad_out, kmap, "feats and grad_out", rows_a=kmap.n_in)
    code = _DT.get(feats.dtype)
    if code is None:
        raise SpconvError(4, f"dtype {feats.dtype} not supported")
    cin, cout = feats.shape[1], grad_out.shape[1]
    shape = (kmap.kernel_volume, cin, cout)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=feats.device)
    elif not (out.is_cuda and out.is_contiguous() and out.dtype == torch.float32 and tuple(out.shape) == shape):
        raise SpconvError(1, "out must be a contiguous fp32 [K^3, C_in, C_out] tensor")
    with _OnDevice(feats.device):
        spconv_backward_weights(feats.data_ptr(), grad_out.data_ptr(), kmap.handle, cin, cout, code, out.data_ptr(),
                                _stream())
    return out


def _forward_operands(feats, weights, kmap: SpconvMap, out):
    """Checks the operands of a forward and returns (c_in, c_out, dtype
    code, out)."""
    global _DT
    torch = _torch()
    if _DT is None:
        _DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if not (feats.is_cuda and weights.is_cuda and feats.is_contiguous() and weights.is_contiguous()):
        raise SpconvError(1, "feats and weights must be contiguous tensors on a HIP device")
    if feats.dim() != 2 or weights.dim() != 3:
        raise SpconvError(1, "feats must be [N, C_in] and weights [K^3, C_in, C_out]")
    n_in, cin = feats.shape
    kv, wcin, cout = weights.shape
    if n_in != kmap.n_in or kv != kmap.kernel_volume or wcin != cin:
        raise SpconvError(1, f"shape mismatch: feats {tuple(feats.shape)}, weights "
                             f"{tuple(weights.shape)}, map n_in={kmap.n_in} K^3={kmap.kernel_volume}")
    dt = feats.dtype
    if weights.dtype != dt:
        raise SpconvError(1, "feats and weights must share one dtype")
    code = _DT.get(dt)
    if code is None:
        raise SpconvError(4, f"dtype {dt} not supported")
    if out is None:
        out = torch.empty((kmap.n, cout), dtype=dt, device=feats.device)
    elif not (out.is_cuda and out.is_contiguous() and out.dtype == dt and tuple(out.shape) == (kmap.n, cout)):
        raise SpconvError(1, "out must be a contiguous [N, C_out] tensor of the feature dtype")
    return cin, cout, code, out


def group_plan(kmap: SpconvMap, epsilon: float, S: float):
    """The offset groups of the adaptive grouping with (epsilon, S) over
    ``kmap``, in execution order (a list of lists of offset indices), and the
    rows of the padded batches."""
    offs, grp, ng, pad = spconv_group_plan(kmap.handle, epsilon, S, kmap.kernel_volume)
    groups = [[] for _ in range(ng)]
    for k, g in zip(offs, grp):
        groups[g].append(k)
    return groups, pad


def group_plan_counts(counts, epsilon: float, S: float, centre: Optional[int] = None):
    """The groups (a list of lists of offset indices, in execution order) and
    padded rows of the adaptive grouping over per-offset map sizes."""
    offs, grp, ng, pad = spconv_group_plan_counts(counts, epsilon, S, -1 if centre is None else centre)
    groups = [[] for _ in range(ng)]
    for k, g in zip(offs, grp):
        groups[g].append(k)
    return groups, pad


def forward_grouped(feats, weights, kmap: SpconvMap, epsilon: float, S: float = float("inf"), out=None):
    """``forward`` in the weight-stationary dataflow with adaptive grouping
    (epsilon, S): gather, one batched MFMA product per group, reduction
    (f16 / bf16, C_in % 32 == 0, C_out % 16 == 0)."""
    cin, cout, code, out = _forward_operands(feats, weights, kmap, out)
    with _OnDevice(feats.device):
        spconv_forward_grouped(feats.data_ptr(), weights.data_ptr(), kmap.handle, cin, cout, code, epsilon, S,
                               out.data_ptr(), _stream())
    return out


def select_dataflow(feats, weights, kmap: SpconvMap, epsilons=None, thresholds=None, reps: int = 3, out=None):
    """Times the fused forward and the grouped forward over a grid of
    (epsilon, S) on these operands and returns (choice, out): choice is a
    dict (dataflow, groups, epsilon, S, ms, fused_ms, candidates) and out
    holds the chosen dataflow's result."""
    cin, cout, code, out = _forward_operands(feats, weights, kmap, out)
    with _OnDevice(feats.device):
        b = spconv_select_dataflow(feats.data_ptr(), weights.data_ptr(), kmap.handle, cin, cout, code, epsilons,
                                   thresholds, reps, out.data_ptr(), _stream())
    choice = {"dataflow": DATAFLOWS.get(b.kind, str(b.kind)), "groups": b.groups, "epsilon": b.epsilon, "S": b.S,
              "ms": b.ms, "fused_ms": b.fused_ms, "candidates": b.candidates}
    return choice, out


def forward_with(choice, feats, weights, kmap: SpconvMap, out=None):
    """The forward in the dataflow ``select_dataflow`` chose."""
    if choice["dataflow"] == "grouped":
        return forward_grouped(feats, weights, kmap, choice["epsilon"], choice["S"], out=out)
    return forward(feats, weights, kmap, out=out)
