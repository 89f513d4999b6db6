"""Decode under HIP graph capture: mp_decode_attn and mp_decode_attn_tables
launch kernels only (no memsets, copies or allocations on the stream), so a
captured step can be replayed.  Each replay runs with new query contents,
with the program's own eager work and synchronisations between replays, and
must equal the eager call on the same query bit for bit."""

import pytest
import torch

import lsh_sampled_sparse_amd as mp
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("tables", [False, True])
def test_captured_decode_replays_match_eager(tables):
    inp = synth.cone_inputs(B=1, H_q=16, H_kv=4, n=9000, d=128, dtype=torch.bfloat16, seeds=[51],
                            device=DEV)
    k, v = inp["k"], inp["v"]
    qs = [synth.cone_inputs(B=1, H_q=16, H_kv=4, n=9000, d=128, dtype=torch.bfloat16,
                            seeds=[60 + i], device=DEV)["q"].contiguous() for i in range(4)]
    idx = mp.build_index(k, 10, 150, 51)
    if tables:
        mp.build_tables(idx)
    decode = mp.decode_attn_tables if tables else mp.decode_attn
    q = qs[0].clone()
    out = torch.empty_like(q)
    scratch = torch.empty(idx.scratch_bytes(16, tables=tables), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        decode(q, idx, k, v, 4, 64, out=out, scratch=scratch, stream=stream)   # warm up
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            decode(q, idx, k, v, 4, 64, out=out, scratch=scratch, stream=stream)
    torch.cuda.synchronize()
    for i, qi in enumerate(qs * 2):
        ref = decode(qi, idx, k, v, 4, 64)           # eager, own scratch
        torch.cuda.synchronize()
        q.copy_(qi)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager decode"
        _ = (k[0, 0, :64].float() @ k[0, 0, :64].float().T).sum().item()   # unrelated eager work
