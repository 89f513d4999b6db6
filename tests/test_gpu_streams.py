"""Calls on a side stream (not torch's current one): the wrappers mark the
buffers they allocate as used by that stream, so the results equal those of
the same calls on the current stream even while the current stream keeps
allocating."""

import pytest
import torch

import lsh_sampled_sparse_amd as mp
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_side_stream_build_and_decode_equal_the_current_stream():
    inp = synth.cone_inputs(B=1, H_q=8, H_kv=2, n=3000, d=128, dtype=torch.bfloat16, seeds=[9],
                            device=DEV)
    k, v, q = inp["k"], inp["v"], inp["q"].contiguous()
    ref_idx = mp.build_index(k, 10, 60, 9)
    mp.build_tables(ref_idx)
    ref = mp.decode_attn(q, ref_idx, k, v, 4, 64)
    ref_t = mp.decode_attn_tables(q, ref_idx, k, v, 4, 64)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    idx = mp.build_index(k, 10, 60, 9, stream=side)
    mp.build_tables(idx, stream=side)
    outs = []
    for i in range(6):
        outs.append(mp.decode_attn(q, idx, k, v, 4, 64, stream=side))
        outs.append(mp.decode_attn_tables(q, idx, k, v, 4, 64, stream=side))
        junk = torch.full((1 << 22,), float(i), device=DEV)   # the current stream allocates
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref if i % 2 == 0 else ref_t), i
