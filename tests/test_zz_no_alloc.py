"""mp_decode_attn_noalloc (scratch in the library's static per-device array)
against mp_decode_attn (caller scratch): bit-identical outputs on two calls
in a row, the second with a smaller input, and a refusal, before any launch,
of a decode whose scratch would not fit the array."""

import pytest
import torch

import lsh_sampled_sparse_amd as mp
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(B, H_q, H_kv, n, dtype, K, L, seed):
    seeds = [seed + 100 * b for b in range(B)]
    inp = synth.cone_inputs(B=B, H_q=H_q, H_kv=H_kv, n=n, d=128, dtype=dtype, seeds=seeds,
                            device=DEV)
    k, v, q = inp["k"], inp["v"], inp["q"].contiguous()
    return k, v, q, mp.build_index(k, K, L, seed)


def _noalloc(q, idx, k, v, n_sink, n_local, out):
    mp.capi.mp_decode_attn_noalloc(q.data_ptr(), q.shape[1], idx.handle, mp.kv_view(k),
                                   mp.kv_view(v), n_sink, n_local, 0.0, out.data_ptr(),
                                   int(torch.cuda.current_stream().cuda_stream))


def test_noalloc_equals_decode_attn_on_two_calls():
    cases = [
        (1, 32, 8, 98304, torch.bfloat16, 10, 150, 2000),   # the 96K layer shape
        (1, 4, 2, 3000, torch.float32, 8, 40, 7),            # then a smaller one
    ]
    for B, H_q, H_kv, n, dtype, K, L, seed in cases:
        print(f"noalloc case n={n} H_q={H_q} {dtype}", flush=True)
        k, v, q, idx = _case(B, H_q, H_kv, n, dtype, K, L, seed)
        ref = mp.decode_attn(q, idx, k, v, 4, 64)
        out = torch.full_like(q, float("nan"))
        _noalloc(q, idx, k, v, 4, 64, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        del k, v, q, idx


def test_noalloc_refuses_scratch_beyond_the_array():
    # 8 sequences x 64 query heads x 157 chunks of partials = 41.8 MB > 32 MiB
    B, H_q, H_kv, n = 8, 64, 8, 80000
    k = torch.zeros(B, H_kv, n, 128, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(B, H_q, 128, device=DEV)
    idx = mp.build_index(k, 1, 2, 3)
    out = torch.zeros_like(q)
    with pytest.raises(mp.MPError, match="MP_E_WORKSPACE.*static scratch"):
        _noalloc(q, idx, k, k, 4, 64, out)
    torch.cuda.synchronize()
    assert not out.any()                                   # nothing ran
