"""Error paths of the C ABI on the GPU, forced from the host so that every
kernel that runs still exits normally:
  * a launch failure (mp_debug_fail_launches) comes back as MP_E_HIP from the
    entry point that made the launch, and the next call works as before;
  * an error an earlier, unrelated HIP call left behind is not reported as a
    later call's failure;
  * a destroyed index handle is refused without being read."""

import ctypes as C

import pytest
import torch

import lsh_sampled_sparse_amd as mp
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(n=1500):
    inp = synth.cone_inputs(B=1, H_q=8, H_kv=2, n=n, d=128, dtype=torch.bfloat16, seeds=[5],
                            device=DEV)
    return inp["k"], inp["v"], inp["q"].contiguous()


def _fail_each_launch(q, idx, k, v, launches):
    ref = mp.decode_attn(q, idx, k, v, 4, 64)
    torch.cuda.synchronize()
    for nth in range(launches):
        mp.capi.mp_debug_fail_launches(nth, 1)
        with pytest.raises(mp.MPError, match="MP_E_HIP"):
            mp.decode_attn(q, idx, k, v, 4, 64)
        torch.cuda.synchronize()
        again = mp.decode_attn(q, idx, k, v, 4, 64)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
    mp.capi.mp_debug_fail_launches(0, 0)


def test_forced_launch_failure_is_mp_e_hip_and_recoverable():
    # 40 chunks a unit (40 records, one a chunk): the query encode, the scan
    # and the merge kernel
    kl, vl, ql = _inputs(40 * 512)
    _fail_each_launch(ql, mp.build_index(kl, 8, 40, 5), kl, vl, 3)
    # 3 records a unit: the merge runs inside the scan, two launches
    k, v, q = _inputs()
    idx = mp.build_index(k, 8, 40, 5)
    _fail_each_launch(q, idx, k, v, 2)
    mp.capi.mp_debug_fail_launches(2, 1)                  # W, mean partial sums, then the mean
    with pytest.raises(mp.MPError, match="MP_E_HIP"):
        mp.build_index(k, 8, 40, 5)
    mp.capi.mp_debug_fail_launches(0, 1)
    with pytest.raises(mp.MPError, match="MP_E_HIP"):
        mp.build_tables(idx)
    mp.capi.mp_debug_fail_launches(0, 0)
    assert idx.tables is None
    with pytest.raises(mp.MPError, match="MP_E_ARG"):           # no tables attached
        mp.decode_attn_tables(q, idx, k, v, 4, 64,
                              scratch=torch.empty(idx.scratch_bytes(8, tables=True),
                                                  dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()


def test_stale_hip_error_is_not_this_calls():
    k, v, q = _inputs()
    idx = mp.build_index(k, 8, 40, 5)
    ref = mp.decode_attn(q, idx, k, v, 4, 64)
    torch.cuda.synchronize()
    hip = C.CDLL("libamdhip64.so")
    hip.hipSetDevice.restype = C.c_int
    hip.hipGetLastError.restype = C.c_int
    out = torch.empty_like(q)
    scr = torch.empty(idx.scratch_bytes(8), dtype=torch.uint8, device=DEV)
    kv_k, kv_v = mp.kv_view(k), mp.kv_view(v)
    sh = int(torch.cuda.current_stream().cuda_stream)
    planted = hip.hipSetDevice(9999)                    # leaves hipErrorInvalidDevice behind
    try:
        assert planted != 0
        # must not report the planted error as its own (and no torch call in
        # between, since torch's launch checks would pick it up)
        mp.capi.mp_decode_attn(q.data_ptr(), 8, idx.handle, kv_k, kv_v, 4, 64, 0.0,
                               out.data_ptr(), scr.data_ptr(), scr.numel(), sh)
    finally:
        pending = hip.hipGetLastError()                 # clear it for torch's own checks
    assert pending == planted                           # it was still there, untouched
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_destroyed_handle_is_refused():
    k, v, q = _inputs()
    idx = mp.build_index(k, 8, 40, 5)
    h = idx.handle
    mp.capi.mp_index_destroy(h)
    idx.handle = None
    scr = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)
    kv = mp.kv_view(k)
    with pytest.raises(mp.MPError, match="MP_E_HANDLE"):
        mp.capi.mp_decode_attn(q.data_ptr(), 8, h, kv, mp.kv_view(v), 4, 64, 0.0, out.data_ptr(),
                               scr.data_ptr(), scr.numel(), 0)
    mp.capi.mp_index_destroy(h)                         # a second destroy is ignored
    assert mp.capi.mp_decode_scratch_bytes(h, 8) == 0
