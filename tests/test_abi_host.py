"""The C ABI surface on the CPU: the library loads, exports every function
include/spconv.h declares, and rejects bad arguments on the host before any
device work (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import submanifold_sparse_convolution_device_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "spconv.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spconv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(sp.EXPORTED)
    L = sp.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_single_hip_runtime_mapped():
    sp.lib()
    assert len(sp._mapped_hip_runtimes()) <= 1


def test_abi_version_and_status_strings():
    assert sp.spconv_abi_version() == 5
    for code, name in sp.STATUS.items():
        assert sp.spconv_status_string(code) == name


def _status_of(fn, *args):
    with pytest.raises(sp.SpconvError) as e:
        fn(*args)
    return e.value.name


def test_build_map_host_validation():
    fake = 4096  # never dereferenced: every case below fails validation first
    assert _status_of(sp.spconv_build_map, 0, 10, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_build_map, fake + 4, 10, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_build_map, fake, 0, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_build_map, fake, -5, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    for K in (0, 2, 4, 9, -1):
        assert _status_of(sp.spconv_build_map, fake, 10, K, 0) == "SPCONV_ERR_UNSUPPORTED"
    assert _status_of(sp.spconv_build_map, fake, (1 << 31) // 27, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert "2^31" in sp.spconv_last_error()
    # out_map NULL
    st = sp.lib().spconv_build_map(fake, 10, 3, 0, None)
    assert sp.STATUS[st] == "SPCONV_ERR_INVALID_ARG"


def test_build_map_async_host_validation():
    """The enqueue-only build rejects the same arguments before any device work."""
    fake = 4096
    b = sp.spconv_build_map_async
    assert _status_of(b, 0, 10, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(b, fake + 8, 10, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(b, fake, 0, 3, 0) == "SPCONV_ERR_INVALID_ARG"
    for K in (0, 2, 8):
        assert _status_of(b, fake, 10, K, 0) == "SPCONV_ERR_UNSUPPORTED"
    assert _status_of(b, fake, (1 << 31) // 343, 7, 0) == "SPCONV_ERR_INVALID_ARG"
    st = sp.lib().spconv_build_map_async(fake, 10, 3, 0, None)
    assert sp.STATUS[st] == "SPCONV_ERR_INVALID_ARG"


def test_forward_host_validation():
    fake = 4096
    fake_map = 8192  # never dereferenced on these error paths
    f = sp.spconv_forward
    # (a NULL feature or output pointer is legal for a map side without rows,
    # so those cases need a real map: tests/test_gpu_grouped.py)
    assert _status_of(f, fake, fake, 0, 32, 32, 1, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake, 0, fake_map, 32, 32, 1, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake + 2, fake, fake_map, 32, 32, 1, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake, fake, fake_map, 32, 32, 7, fake, 0) == "SPCONV_ERR_UNSUPPORTED"
    assert _status_of(f, fake, fake, fake_map, 0, 32, 1, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake, fake, fake_map, 32, 2048, 1, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake, fake, fake_map, 1024, 16, 0, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(f, fake, fake, fake_map, 20, 32, 1, fake, 0) == "SPCONV_ERR_UNSUPPORTED"
    assert _status_of(f, fake, fake, fake_map, 32, 6, 0, fake, 0) == "SPCONV_ERR_UNSUPPORTED"


def test_grouped_host_validation():
    """The grouped forward, its plan and the selector reject bad arguments
    before they read the map or touch the device."""
    fake, fake_map = 4096, 8192
    g = sp.spconv_forward_grouped
    assert _status_of(g, fake, fake, 0, 32, 32, 1, 0.1, 1e9, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(g, fake, 0, fake_map, 32, 32, 1, 0.1, 1e9, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(g, fake, fake, fake_map, 32, 32, 7, 0.1, 1e9, fake, 0) == "SPCONV_ERR_UNSUPPORTED"
    assert _status_of(sp.spconv_group_plan, 0, 0.1, 1e9, 27) == "SPCONV_ERR_INVALID_ARG"
    sel = sp.spconv_select_dataflow
    assert _status_of(sel, fake, fake, 0, 32, 32, 1, None, None, 3, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sel, fake, fake, fake_map, 32, 32, 9, None, None, 3, fake, 0) == "SPCONV_ERR_UNSUPPORTED"


def test_prepared_weights_host_validation():
    """Weight preparation and the prepared forward reject bad arguments
    before any device work."""
    fake = 4096
    p = sp.spconv_weights_prepare
    assert _status_of(p, 0, 27, 32, 32, 1, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(p, fake + 8, 27, 32, 32, 1, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(p, fake, 27, 32, 32, 7, 0) == "SPCONV_ERR_UNSUPPORTED"
    for kv in (0, 344, -1):
        assert _status_of(p, fake, kv, 32, 32, 1, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(p, fake, 27, 0, 32, 1, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(p, fake, 27, 32, 2048, 1, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(p, fake, 27, 20, 32, 1, 0) == "SPCONV_ERR_UNSUPPORTED"
    st = sp.lib().spconv_weights_prepare(fake, 27, 32, 32, 1, None, None)
    assert sp.STATUS[st] == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_forward_prepared, fake, 0, 8192, fake, 0) == "SPCONV_ERR_INVALID_ARG"
    sp.spconv_weights_free(0)  # NULL is ignored


def test_map_queries_reject_null():
    assert _status_of(sp.spconv_map_wait, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_map_info, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_map_lists, 0) == "SPCONV_ERR_INVALID_ARG"
    assert _status_of(sp.spconv_map_counts, 0, 27) == "SPCONV_ERR_INVALID_ARG"
    sp.spconv_map_free(0)  # NULL is ignored


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(sp, "_LIB", None)
    monkeypatch.setattr(sp, "LIB_PATH", str(tmp_path / "libspconv.so"))
    with pytest.raises(RuntimeError, match="not built"):
        sp.lib()
