"""ctypes binding of libmagicpig (include/magicpig.h), same names as the C ABI.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libmagicpig.so.  If the library is missing this module raises; there
is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmagicpig.so")

MP_OK, MP_E_ARG, MP_E_SHAPE, MP_E_DTYPE, MP_E_WORKSPACE, MP_E_HIP, MP_E_HANDLE = range(7)
MP_F32, MP_BF16 = 0, 1
MP_CHUNK = 512
MP_INDEX_MIPS = 1

EXPORTED = [
    "mp_index_workspace_bytes", "mp_build_index", "mp_decode_scratch_bytes", "mp_decode_attn",
    "mp_decode_attn_timed", "mp_decode_debug", "mp_index_views", "mp_index_destroy", "mp_status_str", "mp_last_error",
    "mp_tables_workspace_bytes", "mp_build_tables", "mp_decode_tables_scratch_bytes",
    "mp_decode_attn_tables", "mp_decode_attn_tables_timed", "mp_decode_tables_debug",
    "mp_tables_views", "mp_build_index_cap", "mp_index_append", "mp_index_workspace_bytes_ex",
    "mp_build_index_ex", "mp_index_lift_views", "mp_stream_read", "mp_debug_fail_launches",
    "mp_decode_attn_noalloc", "mp_decode_attn_append",
]


class mp_kv_view(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("B", C.c_int32), ("H", C.c_int32),
                ("n", C.c_int32), ("d", C.c_int32), ("stride_b", C.c_int64),
                ("stride_h", C.c_int64), ("stride_n", C.c_int64)]


class MPError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {mp_status_str(status)} ({detail})")


_lib = None


def lib():
    """Load libmagicpig.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime (same soname) then serves this library too,
        # so torch's streams and events are valid handles here.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m lsh_sampled_sparse_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.mp_index_workspace_bytes.restype = sz
        L.mp_index_workspace_bytes.argtypes = [i32] * 6
        L.mp_build_index.restype = C.c_int
        L.mp_build_index.argtypes = [C.POINTER(mp_kv_view), i32, i32, C.c_uint64, vp, sz, vp,
                                     C.POINTER(vp)]
        L.mp_build_index_cap.restype = C.c_int
        L.mp_build_index_cap.argtypes = [C.POINTER(mp_kv_view), i32, i32, C.c_uint64, i32, vp, sz,
                                         vp, C.POINTER(vp)]
        L.mp_index_workspace_bytes_ex.restype = sz
        L.mp_index_workspace_bytes_ex.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.mp_build_index_ex.restype = C.c_int
        L.mp_build_index_ex.argtypes = [C.POINTER(mp_kv_view), i32, i32, C.c_uint64, i32, i32, vp,
                                        sz, vp, C.POINTER(vp)]
        L.mp_index_lift_views.restype = C.c_int
        L.mp_index_lift_views.argtypes = [vp, C.POINTER(vp), C.POINTER(vp)]
        L.mp_stream_read.restype = C.c_int
        L.mp_stream_read.argtypes = [vp, C.c_int64, vp, i32, vp]
        L.mp_index_append.restype = C.c_int
        L.mp_index_append.argtypes = [vp, C.POINTER(mp_kv_view), vp]
        L.mp_decode_scratch_bytes.restype = sz
        L.mp_decode_scratch_bytes.argtypes = [vp, i32]
        dec = [vp, i32, vp, C.POINTER(mp_kv_view), C.POINTER(mp_kv_view), i32, i32, C.c_float,
               vp, vp, sz, vp]
        L.mp_decode_attn.restype = C.c_int
        L.mp_decode_attn.argtypes = dec
        L.mp_decode_attn_append.restype = C.c_int
        L.mp_decode_attn_append.argtypes = dec
        L.mp_decode_attn_noalloc.restype = C.c_int
        L.mp_decode_attn_noalloc.argtypes = [vp, i32, vp, C.POINTER(mp_kv_view),
                                             C.POINTER(mp_kv_view), i32, i32, C.c_float, vp, vp]
        L.mp_decode_attn_timed.restype = C.c_int
        L.mp_decode_attn_timed.argtypes = dec + [vp, vp]
        L.mp_decode_debug.restype = C.c_int
        L.mp_decode_debug.argtypes = dec + [vp, vp, vp, vp]
        L.mp_tables_workspace_bytes.restype = sz
        L.mp_tables_workspace_bytes.argtypes = [vp]
        L.mp_build_tables.restype = C.c_int
        L.mp_build_tables.argtypes = [vp, vp, sz, vp]
        L.mp_decode_tables_scratch_bytes.restype = sz
        L.mp_decode_tables_scratch_bytes.argtypes = [vp, i32]
        L.mp_decode_attn_tables.restype = C.c_int
        L.mp_decode_attn_tables.argtypes = dec
        L.mp_decode_attn_tables_timed.restype = C.c_int
        L.mp_decode_attn_tables_timed.argtypes = dec + [vp, vp]
        L.mp_decode_tables_debug.restype = C.c_int
        L.mp_decode_tables_debug.argtypes = dec + [vp, vp, vp, vp]
        L.mp_tables_views.restype = C.c_int
        L.mp_tables_views.argtypes = [vp, C.POINTER(vp), C.POINTER(vp)]
        L.mp_index_views.restype = C.c_int
        L.mp_index_views.argtypes = [vp, C.POINTER(vp), C.POINTER(vp), C.POINTER(vp),
                                     C.POINTER(i32)]
        L.mp_index_destroy.restype = None
        L.mp_index_destroy.argtypes = [vp]
        L.mp_status_str.restype = C.c_char_p
        L.mp_status_str.argtypes = [C.c_int]
        L.mp_last_error.restype = C.c_char_p
        L.mp_last_error.argtypes = []
        L.mp_debug_fail_launches.restype = None
        L.mp_debug_fail_launches.argtypes = [i32, i32]
        _lib = L
    return _lib


def mp_status_str(status: int) -> str:
    return lib().mp_status_str(status).decode()


def mp_last_error() -> str:
    return lib().mp_last_error().decode()


def _check(status: int, func: str):
    if status != MP_OK:
        raise MPError(status, func, mp_last_error())


def mp_index_workspace_bytes(B, H_kv, n, d, K, L) -> int:
    return int(lib().mp_index_workspace_bytes(B, H_kv, n, d, K, L))


def mp_build_index(keys: mp_kv_view, K: int, L: int, seed: int, workspace: int,
                   workspace_bytes: int, stream: int) -> int:
    """Returns the index handle (an int); raises MPError on a non-OK status."""
    out = C.c_void_p()
    st = lib().mp_build_index(C.byref(keys), K, L, seed & (2**64 - 1), workspace,
                              workspace_bytes, stream, C.byref(out))
    _check(st, "mp_build_index")
    return out.value


def mp_build_index_cap(keys: mp_kv_view, K: int, L: int, seed: int, n_cap: int, workspace: int,
                       workspace_bytes: int, stream: int) -> int:
    """mp_build_index with room to grow to n_cap keys; returns the handle."""
    out = C.c_void_p()
    st = lib().mp_build_index_cap(C.byref(keys), K, L, seed & (2**64 - 1), n_cap, workspace,
                                  workspace_bytes, stream, C.byref(out))
    _check(st, "mp_build_index_cap")
    return out.value


def mp_index_workspace_bytes_ex(B, H_kv, n, d, K, L, flags) -> int:
    return int(lib().mp_index_workspace_bytes_ex(B, H_kv, n, d, K, L, flags))


def mp_build_index_ex(keys: mp_kv_view, K: int, L: int, seed: int, n_cap: int, flags: int,
                      workspace: int, workspace_bytes: int, stream: int) -> int:
    """mp_build_index_cap with build flags (MP_INDEX_*); returns the handle."""
    out = C.c_void_p()
    st = lib().mp_build_index_ex(C.byref(keys), K, L, seed & (2**64 - 1), n_cap, flags, workspace,
                                 workspace_bytes, stream, C.byref(out))
    _check(st, "mp_build_index_ex")
    return out.value


def mp_index_lift_views(idx: int):
    w, r = C.c_void_p(), C.c_void_p()
    _check(lib().mp_index_lift_views(idx, C.byref(w), C.byref(r)), "mp_index_lift_views")
    return w.value, r.value


def mp_stream_read(data: int, nbytes: int, sink: int, blocks: int, stream: int) -> None:
    _check(lib().mp_stream_read(data, nbytes, sink, blocks, stream), "mp_stream_read")


def mp_index_append(idx: int, keys: mp_kv_view, stream: int) -> None:
    _check(lib().mp_index_append(idx, C.byref(keys), stream), "mp_index_append")


def mp_decode_scratch_bytes(idx: int, H_q: int) -> int:
    return int(lib().mp_decode_scratch_bytes(idx, H_q))


def mp_decode_attn(q: int, H_q: int, idx: int, k: mp_kv_view, v: mp_kv_view, n_sink: int,
                   n_local: int, scale: float, out: int, scratch: int, scratch_bytes: int,
                   stream: int) -> None:
    st = lib().mp_decode_attn(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale, out,
                              scratch, scratch_bytes, stream)
    _check(st, "mp_decode_attn")


def mp_decode_attn_append(q: int, H_q: int, idx: int, k: mp_kv_view, v: mp_kv_view, n_sink: int,
                          n_local: int, scale: float, out: int, scratch: int, scratch_bytes: int,
                          stream: int) -> None:
    st = lib().mp_decode_attn_append(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale,
                                     out, scratch, scratch_bytes, stream)
    _check(st, "mp_decode_attn_append")


def mp_decode_attn_noalloc(q: int, H_q: int, idx: int, k: mp_kv_view, v: mp_kv_view,
                           n_sink: int, n_local: int, scale: float, out: int, stream: int) -> None:
    st = lib().mp_decode_attn_noalloc(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale,
                                      out, stream)
    _check(st, "mp_decode_attn_noalloc")


def mp_decode_attn_timed(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, ev_scan_begin, ev_scan_end) -> None:
    st = lib().mp_decode_attn_timed(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale,
                                    out, scratch, scratch_bytes, stream, ev_scan_begin,
                                    ev_scan_end)
    _check(st, "mp_decode_attn_timed")


def mp_decode_debug(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                    stream, qcodes, counts, s_idx, s_len) -> None:
    st = lib().mp_decode_debug(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale, out,
                               scratch, scratch_bytes, stream, qcodes, counts, s_idx, s_len)
    _check(st, "mp_decode_debug")


def mp_tables_workspace_bytes(idx: int) -> int:
    return int(lib().mp_tables_workspace_bytes(idx))


def mp_build_tables(idx: int, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check(lib().mp_build_tables(idx, workspace, workspace_bytes, stream), "mp_build_tables")


def mp_decode_tables_scratch_bytes(idx: int, H_q: int) -> int:
    return int(lib().mp_decode_tables_scratch_bytes(idx, H_q))


def mp_decode_attn_tables(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                          stream) -> None:
    st = lib().mp_decode_attn_tables(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local, scale,
                                     out, scratch, scratch_bytes, stream)
    _check(st, "mp_decode_attn_tables")


def mp_decode_attn_tables_timed(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch,
                                scratch_bytes, stream, ev_gather_begin, ev_gather_end) -> None:
    st = lib().mp_decode_attn_tables_timed(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local,
                                           scale, out, scratch, scratch_bytes, stream,
                                           ev_gather_begin, ev_gather_end)
    _check(st, "mp_decode_attn_tables_timed")


def mp_decode_tables_debug(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch,
                           scratch_bytes, stream, qcodes, counts2, s_idx, s_len) -> None:
    st = lib().mp_decode_tables_debug(q, H_q, idx, C.byref(k), C.byref(v), n_sink, n_local,
                                      scale, out, scratch, scratch_bytes, stream, qcodes, counts2,
                                      s_idx, s_len)
    _check(st, "mp_decode_tables_debug")


def mp_tables_views(idx: int):
    off, ent = C.c_void_p(), C.c_void_p()
    _check(lib().mp_tables_views(idx, C.byref(off), C.byref(ent)), "mp_tables_views")
    return off.value, ent.value


def mp_index_views(idx: int):
    W, mu, codes = C.c_void_p(), C.c_void_p(), C.c_void_p()
    n_pad = C.c_int32()
    st = lib().mp_index_views(idx, C.byref(W), C.byref(mu), C.byref(codes), C.byref(n_pad))
    _check(st, "mp_index_views")
    return W.value, mu.value, codes.value, n_pad.value


def mp_index_destroy(idx) -> None:
    lib().mp_index_destroy(idx)


def mp_debug_fail_launches(skip: int, count: int) -> None:
    """Test aid: after `skip` launches, the next `count` fail (magicpig_testing.h)."""
    lib().mp_debug_fail_launches(skip, count)
