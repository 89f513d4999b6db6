"""The C ABI library loads, exports every function include/magicpig.h declares,
and rejects bad arguments on the host before touching the GPU (CPU only: no
compute call is made)."""

import ctypes as C
import os
import re

import pytest

from lsh_sampled_sparse_amd import capi

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(mp_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = capi.lib()
    names = _declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(capi.EXPORTED)


def test_status_strings():
    for s in range(7):
        assert capi.mp_status_str(s).startswith("MP_")
    assert "unknown" in capi.mp_status_str(99)


def test_workspace_bytes_rejects_bad_sizes_and_covers_codes():
    f = capi.mp_index_workspace_bytes
    assert f(1, 8, 98304, 64, 10, 150) == 0       # d != 128
    assert f(1, 8, 98304, 128, 17, 150) == 0      # K > 16
    assert f(1, 8, 98304, 128, 10, 1) == 0        # L < 2
    assert f(1, 8, 98304, 128, 10, 256) == 0      # L > 255
    assert f(0, 8, 98304, 128, 10, 150) == 0
    assert f(1, 8, 0, 128, 10, 150) == 0
    a = f(1, 8, 98304, 128, 10, 150)
    codes = 8 * 98304 * 150 * 10 // 8            # K = 10 bits per key and table
    assert codes <= a < codes + (8 << 20) and a % 256 == 0
    assert f(1, 8, 98305, 128, 10, 150) > a                 # ragged tail pads a chunk
    assert f(1, 8, 1, 128, 0, 2) > 0                         # K = 0 is allowed


def _view(**kw):
    v = dict(data=0x10000, dtype=capi.MP_BF16, B=1, H=2, n=1000, d=128, stride_b=2 * 1000 * 128,
             stride_h=1000 * 128, stride_n=128)
    v.update(kw)
    return capi.mp_kv_view(**v)


@pytest.mark.parametrize("kw,K,L,status", [
    (dict(data=None), 10, 150, capi.MP_E_ARG),
    (dict(dtype=7), 10, 150, capi.MP_E_DTYPE),
    (dict(d=64), 10, 150, capi.MP_E_SHAPE),
    (dict(n=0), 10, 150, capi.MP_E_SHAPE),
    (dict(stride_n=100), 10, 150, capi.MP_E_SHAPE),
    (dict(data=0x10002), 10, 150, capi.MP_E_SHAPE),      # misaligned rows
    (dict(stride_n=129), 10, 150, capi.MP_E_SHAPE),      # 258-byte bf16 rows
    (dict(), 17, 150, capi.MP_E_ARG),
    (dict(), -1, 150, capi.MP_E_ARG),
    (dict(), 10, 1, capi.MP_E_ARG),
    (dict(), 10, 300, capi.MP_E_ARG),
])
def test_build_index_rejects_bad_arguments(kw, K, L, status):
    out = C.c_void_p(123)
    st = capi.lib().mp_build_index(C.byref(_view(**kw)), K, L, 0, 0x100000, 1 << 40, None,
                                   C.byref(out))
    assert st == status, capi.mp_last_error()
    assert out.value is None
    assert capi.mp_last_error() != ""


def test_build_index_rejects_bad_workspace():
    out = C.c_void_p()
    v = _view()
    need = capi.mp_index_workspace_bytes(1, 2, 1000, 128, 10, 150)
    L = capi.lib()
    assert L.mp_build_index(C.byref(v), 10, 150, 0, None, need, None, C.byref(out)) == capi.MP_E_WORKSPACE
    assert L.mp_build_index(C.byref(v), 10, 150, 0, 0x100010, need, None, C.byref(out)) == capi.MP_E_WORKSPACE
    assert L.mp_build_index(C.byref(v), 10, 150, 0, 0x100000, need - 1, None, C.byref(out)) == capi.MP_E_WORKSPACE
    assert "needed" in capi.mp_last_error()
    assert L.mp_build_index(C.byref(v), 10, 150, 0, 0x100000, need, None, None) == capi.MP_E_ARG


def test_decode_rejects_dead_handles():
    L = capi.lib()
    fake = (C.c_uint8 * 4096)()          # zeroed host memory: no magic number
    v = _view()
    for h in (None, C.addressof(fake)):
        st = L.mp_decode_attn(0x1000, 8, h, C.byref(v), C.byref(v), 4, 64, 0.0, 0x2000, 0x3000,
                              1 << 30, None)
        assert st == capi.MP_E_HANDLE
    assert capi.mp_decode_scratch_bytes(None, 8) == 0
    assert capi.mp_decode_scratch_bytes(C.addressof(fake), 8) == 0
    W, mu, codes, n_pad = C.c_void_p(), C.c_void_p(), C.c_void_p(), C.c_int32()
    assert L.mp_index_views(None, C.byref(W), C.byref(mu), C.byref(codes), C.byref(n_pad)) == capi.MP_E_HANDLE
    L.mp_index_destroy(None)            # ignored


def test_python_layer_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    monkeypatch.setattr(capi, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(capi, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        capi.lib()


def test_tables_calls_reject_a_dead_handle():
    """The bucketed-table calls check the index handle on the host."""
    assert capi.mp_tables_workspace_bytes(None) == 0
    assert capi.mp_decode_tables_scratch_bytes(None, 32) == 0
    with pytest.raises(capi.MPError, match="MP_E_HANDLE"):
        capi.mp_build_tables(None, None, 0, None)
    with pytest.raises(capi.MPError, match="MP_E_HANDLE"):
        capi.mp_tables_views(None)


def test_capacity_build_and_append_check_their_arguments_on_the_host():
    """mp_build_index_cap refuses a capacity below the key count or above the
    size limits before touching the device; mp_index_append refuses a dead
    handle."""
    L = capi.lib()
    out = C.c_void_p(123)
    v = _view()                                   # n = 1000 keys
    need = capi.mp_index_workspace_bytes(1, 2, 4000, 128, 10, 150)
    assert need > capi.mp_index_workspace_bytes(1, 2, 1000, 128, 10, 150)
    for cap in (999, 0, -5):
        st = L.mp_build_index_cap(C.byref(v), 10, 150, 0, cap, 0x100000, need, None, C.byref(out))
        assert st == capi.MP_E_ARG, capi.mp_last_error()
        assert out.value is None
    assert "capacity" in capi.mp_last_error()
    st = L.mp_build_index_cap(C.byref(v), 10, 150, 0, 4000, 0x100000, need - 1, None, C.byref(out))
    assert st == capi.MP_E_WORKSPACE
    fake = (C.c_uint8 * 4096)()
    for h in (None, C.addressof(fake)):
        assert L.mp_index_append(h, C.byref(v), None) == capi.MP_E_HANDLE
    with pytest.raises(capi.MPError, match="MP_E_HANDLE"):
        capi.mp_index_append(None, v, 0)


def test_lift_build_checks_flags_and_sizes_on_the_host():
    f = capi.mp_index_workspace_bytes_ex
    plain = f(1, 8, 98304, 128, 10, 150, 0)
    lifted = f(1, 8, 98304, 128, 10, 150, capi.MP_INDEX_MIPS)
    assert plain == capi.mp_index_workspace_bytes(1, 8, 98304, 128, 10, 150)
    # the lift adds the fp64 key norms (8 B per key) and small per-unit arrays
    assert 8 * 98304 * 8 <= lifted - plain < 8 * 98304 * 8 + (1 << 20)
    assert f(1, 8, 98304, 128, 10, 150, 2) == 0                  # unknown flag
    L = capi.lib()
    out = C.c_void_p(123)
    v = _view()
    need = f(1, 2, 1000, 128, 10, 150, capi.MP_INDEX_MIPS)
    st = L.mp_build_index_ex(C.byref(v), 10, 150, 0, 1000, 6, 0x100000, need, None, C.byref(out))
    assert st == capi.MP_E_ARG and "flags" in capi.mp_last_error()
    st = L.mp_build_index_ex(C.byref(v), 10, 150, 0, 1000, capi.MP_INDEX_MIPS, 0x100000, need - 1,
                             None, C.byref(out))
    assert st == capi.MP_E_WORKSPACE
    with pytest.raises(capi.MPError, match="MP_E_HANDLE"):
        capi.mp_index_lift_views(None)


def test_stream_read_probe_checks_arguments_on_the_host():
    L = capi.lib()
    assert L.mp_stream_read(None, 1 << 20, 0x2000, 1024, None) == capi.MP_E_ARG
    assert L.mp_stream_read(0x1000, 8, 0x2000, 1024, None) == capi.MP_E_ARG
    assert L.mp_stream_read(0x1004, 1 << 20, 0x2000, 1024, None) == capi.MP_E_ARG
    assert L.mp_stream_read(0x1000, 1 << 20, None, 1024, None) == capi.MP_E_ARG
    assert L.mp_stream_read(0x1000, 1 << 20, 0x2000, 0, None) == capi.MP_E_ARG
