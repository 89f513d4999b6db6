"""MI355X-native MagicPIG decode attention (LSH-sampled sparse attention).

PyTorch supplies device memory and streams; every step of the path runs in the
HIP kernels of ``libmagicpig.so`` behind the C ABI in ``include/magicpig.h``.
This module only marshals tensors into that ABI (see ``capi`` for the
one-to-one ctypes binding).

    idx = build_index(keys, K=10, L=150, seed=2000)          # keys [B][H_kv][n][128]
    out = decode_attn(q, idx, keys, values, n_sink=4, n_local=64)   # q [B][H_q][128] fp32
"""

from __future__ import annotations

import torch

from . import capi
from .capi import MPError, MP_CHUNK

__all__ = ["MagicPIGIndex", "build_index", "build_tables", "append_index", "decode_attn",
           "decode_attn_append", "decode_debug", "decode_attn_tables", "decode_tables_debug",
           "kv_view", "capi", "MPError", "MP_CHUNK"]

_DTYPES = {torch.float32: capi.MP_F32, torch.bfloat16: capi.MP_BF16}


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _side_stream(stream, device):
    """The torch stream object of `stream` (a torch stream or a raw
    hipStream_t handle) when it is not the current stream of `device`, else
    None: the library enqueues on the stream it is given, while the tensors
    made here come from torch's caching allocator on the current stream."""
    if stream is None:
        return None
    cur = torch.cuda.current_stream(device)
    h = _stream(stream)
    if h == int(cur.cuda_stream):
        return None
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(h, device=device)


def _keep_alive_on(side, *tensors):
    """Mark tensors as used by work on the side stream, so that the caching
    allocator does not hand their memory out again (after they are freed here)
    before that work has run."""
    if side is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(side)


def kv_view(t: torch.Tensor) -> capi.mp_kv_view:
    """mp_kv_view of a [B][H][n][128] device tensor (fp32 or bf16, last dim contiguous)."""
    if t.dim() != 4:
        raise ValueError("expected a [B][H][n][d] tensor")
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if t.stride(3) != 1:
        raise ValueError("the d axis must be contiguous")
    B, H, n, d = t.shape
    return capi.mp_kv_view(t.data_ptr(), _DTYPES[t.dtype], B, H, n, d, t.stride(0), t.stride(1),
                           t.stride(2))


class MagicPIGIndex:
    """A built index: the host handle plus the device workspace that holds
    W, mu and the key codes (as bit planes)."""

    def __init__(self, handle: int, workspace: torch.Tensor, keys_shape, K: int, L: int,
                 seed: int, dtype, capacity: int = 0, mips: bool = False):
        self.handle = handle
        self.workspace = workspace
        self.B, self.H_kv, self.n, self.d = keys_shape
        self.capacity = max(capacity, self.n)
        self.mips = mips
        self.K, self.L, self.seed, self.dtype = K, L, seed, dtype
        self.tables = None      # table workspace, once build_tables ran

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self.handle = None
            try:
                capi.mp_index_destroy(h)
            except Exception:          # interpreter teardown: module globals already gone
                pass

    def _slice(self, ptr, numel, dtype):
        base = self.workspace.data_ptr()
        off = ptr - base
        esz = torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + numel * esz].view(dtype)

    def views(self):
        """Device tensors aliasing the workspace: W [R][128] fp32, mu [B][H_kv][128]
        fp32 and the key codes as bit planes [B][H_kv][n_pad/512][L*Kr][16]
        uint32 (as int32 storage), Kr = max(K, 1): bit j of word w of row
        l*Kr + b of chunk c is bit b of the table-l code of key 512c + 32w + j."""
        W, mu, planes, n_pad = capi.mp_index_views(self.handle)
        R = self.K * self.L
        Wt = self._slice(W, R * 128, torch.float32).view(R, 128)
        mut = self._slice(mu, self.B * self.H_kv * 128, torch.float32).view(self.B, self.H_kv, 128)
        nc = n_pad // MP_CHUNK
        nc_cap = -(-self.capacity // MP_CHUNK)       # chunks between units
        rows = self.L * max(self.K, 1)
        words = MP_CHUNK // 32
        pt = self._slice(planes, self.B * self.H_kv * nc_cap * rows * words, torch.int32)
        return Wt, mut, pt.view(self.B, self.H_kv, nc_cap, rows, words)[:, :, :nc]

    def lift_views(self):
        """The lift of an index built with mips=True: the hyperplanes' extra
        coordinate [K*L] and the radius r of each unit [B][H_kv] (fp32)."""
        w, r = capi.mp_index_lift_views(self.handle)
        R = self.K * self.L
        return (self._slice(w, R, torch.float32),
                self._slice(r, self.B * self.H_kv, torch.float32).view(self.B, self.H_kv))

    def scratch_bytes(self, H_q: int, tables: bool = False) -> int:
        if tables:
            return capi.mp_decode_tables_scratch_bytes(self.handle, H_q)
        return capi.mp_decode_scratch_bytes(self.handle, H_q)

    def table_views(self):
        """Device tensors aliasing the table workspace: offsets
        [B][H_kv][L][2^K + 1] and entries [B][H_kv][L][n] (uint32 as int32)."""
        off, ent = capi.mp_tables_views(self.handle)
        nb = (1 << self.K) + 1
        o = self._slice_of(self.tables, off, self.B * self.H_kv * self.L * nb, torch.int32)
        e = self._slice_of(self.tables, ent, self.B * self.H_kv * self.L * self.n, torch.int32)
        return (o.view(self.B, self.H_kv, self.L, nb), e.view(self.B, self.H_kv, self.L, self.n))

    @staticmethod
    def _slice_of(buf, ptr, numel, dtype):
        off = ptr - buf.data_ptr()
        esz = torch.empty(0, dtype=dtype).element_size()
        return buf[off:off + numel * esz].view(dtype)


def build_index(keys: torch.Tensor, K: int, L: int, seed: int, stream=None,
                capacity: int | None = None, mips: bool = False) -> MagicPIGIndex:
    """Index of `keys` [B][H_kv][n][128]; with `capacity` (>= n) it can later
    grow to that many keys by append_index (see mp_build_index_cap); with
    mips=True keys are lifted to a sphere before hashing (MP_INDEX_MIPS)."""
    view = kv_view(keys)
    n_cap = view.n if capacity is None else capacity
    flags = capi.MP_INDEX_MIPS if mips else 0
    nbytes = capi.mp_index_workspace_bytes_ex(view.B, view.H, n_cap, view.d, K, L, flags)
    if nbytes == 0:
        raise ValueError(f"invalid index sizes B={view.B} H={view.H} n={n_cap} d={view.d} "
                         f"K={K} L={L}")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=keys.device)
    _keep_alive_on(_side_stream(stream, keys.device), ws)
    if mips:
        h = capi.mp_build_index_ex(view, K, L, seed, n_cap, flags, ws.data_ptr(), nbytes,
                                   _stream(stream))
    elif capacity is None:
        h = capi.mp_build_index(view, K, L, seed, ws.data_ptr(), nbytes, _stream(stream))
    else:
        h = capi.mp_build_index_cap(view, K, L, seed, n_cap, ws.data_ptr(), nbytes,
                                    _stream(stream))
    return MagicPIGIndex(h, ws, tuple(keys.shape), K, L, seed, keys.dtype, n_cap, mips)


def append_index(index: MagicPIGIndex, keys: torch.Tensor, stream=None) -> MagicPIGIndex:
    """Grow `index` to the keys of `keys` [B][H_kv][n_new][128], whose first
    index.n keys are the indexed ones (see mp_index_append).  Detaches any
    bucketed tables."""
    capi.mp_index_append(index.handle, kv_view(keys), _stream(stream))
    index.n = keys.shape[2]
    # decodes on other streams may still read the old tables: they were marked
    # on those streams when the decode was enqueued (see _decode)
    index.tables = None
    return index


def build_tables(index: MagicPIGIndex, stream=None) -> MagicPIGIndex:
    """Build the bucketed hash tables of `index` (see mp_build_tables); the
    table workspace is kept on the index object."""
    nbytes = capi.mp_tables_workspace_bytes(index.handle)
    if nbytes == 0:
        raise ValueError(f"this index cannot have tables (K={index.K}, n={index.n})")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=index.workspace.device)
    _keep_alive_on(_side_stream(stream, ws.device), ws)
    capi.mp_build_tables(index.handle, ws.data_ptr(), nbytes, _stream(stream))
    index.tables = ws
    return index


def _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, debug, tables=False,
            append=False):
    if q.dtype != torch.float32 or not q.is_contiguous() or q.dim() != 3:
        raise ValueError("q must be a contiguous [B][H_q][128] float32 tensor")
    B, H_q, d = q.shape
    if out is None:
        out = torch.empty(B, H_q, d, dtype=torch.float32, device=q.device)
    need = index.scratch_bytes(H_q, tables)
    if need == 0:
        raise ValueError(f"H_q={H_q} does not fit the index (H_kv={index.H_kv})")
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.uint8, device=q.device)
    kv_k, kv_v = kv_view(k), kv_view(v)
    s = _stream(stream)
    # on a side stream, the buffers allocated here and the index's workspaces
    # must outlive this call's kernels, not just this Python call
    _keep_alive_on(_side_stream(stream, q.device), out, scratch, index.workspace,
                   index.tables if tables else None)
    if append:
        capi.mp_decode_attn_append(q.data_ptr(), H_q, index.handle, kv_k, kv_v, n_sink, n_local,
                                   float(scale), out.data_ptr(), scratch.data_ptr(),
                                   scratch.numel(), s)
        index.n = k.shape[2]
        # decodes on other streams may still read the old tables: they were
        # marked on those streams when the decode was enqueued
        index.tables = None
        return out
    if not debug:
        f = capi.mp_decode_attn_tables if tables else capi.mp_decode_attn
        f(q.data_ptr(), H_q, index.handle, kv_k, kv_v, n_sink, n_local, float(scale),
          out.data_ptr(), scratch.data_ptr(), scratch.numel(), s)
        return out
    n = index.n
    qcodes = torch.empty(B, H_q, index.L, dtype=torch.int16, device=q.device)
    counts = torch.empty(B, H_q, n, dtype=torch.uint8, device=q.device)
    s_idx = torch.empty(B, H_q, n, dtype=torch.int32, device=q.device)
    s_len = torch.empty(B, H_q, dtype=torch.int32, device=q.device)
    _keep_alive_on(_side_stream(stream, q.device), qcodes, counts, s_idx, s_len)
    f = capi.mp_decode_tables_debug if tables else capi.mp_decode_debug
    f(q.data_ptr(), H_q, index.handle, kv_k, kv_v, n_sink, n_local, float(scale), out.data_ptr(),
      scratch.data_ptr(), scratch.numel(), s, qcodes.data_ptr(), counts.data_ptr(),
      s_idx.data_ptr(), s_len.data_ptr())
    return dict(out=out, qcodes=qcodes, counts=counts, s_idx=s_idx, s_len=s_len)


def decode_attn(q, index, k, v, n_sink, n_local, scale=0.0, out=None, scratch=None, stream=None):
    """One decode step: out [B][H_q][128] fp32 (see mp_decode_attn)."""
    return _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, False)


def decode_attn_append(q, index, k, v, n_sink, n_local, scale=0.0, out=None, scratch=None,
                       stream=None):
    """Grow `index` to the keys of k [B][H_kv][n_new][128] and decode over
    them in one call (see mp_decode_attn_append): out [B][H_q][128] fp32.
    Detaches any bucketed tables."""
    return _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, False,
                   append=True)


def decode_debug(q, index, k, v, n_sink, n_local, scale=0.0, out=None, scratch=None,
                 stream=None):
    """decode_attn plus qcodes, counts, s_idx, s_len (see mp_decode_debug)."""
    return _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, True)


def decode_attn_tables(q, index, k, v, n_sink, n_local, scale=0.0, out=None, scratch=None,
                       stream=None):
    """decode_attn through the bucketed tables (see mp_decode_attn_tables)."""
    return _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, False, True)


def decode_tables_debug(q, index, k, v, n_sink, n_local, scale=0.0, out=None, scratch=None,
                        stream=None):
    """decode_attn_tables plus qcodes, counts (min(count, 2)), s_idx, s_len."""
    return _decode(q, index, k, v, n_sink, n_local, scale, out, scratch, stream, True, True)
