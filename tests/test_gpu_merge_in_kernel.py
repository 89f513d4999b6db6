"""The merge inside the gather kernels, step after step.

Where a unit has few records, the workgroup that stores a unit's last
record merges them all in the same kernel: the records go out with
device-scope stores, are counted once those have completed, and are read
back with device-scope loads by a workgroup that may sit on another XCD.
The fold runs in record order, so a decode of the same inputs gives the same
bits every time.  These tests repeat such decodes many times, with the
scratch reused and the inputs alternating, and require every output to equal
the first one bit for bit: a record read before it was visible would change
the bits.  The 16K workload's shape (8 units of 32 chunks; the scan's runs
of one chunk and the table path's chunks both give 32 records a unit) and
a batch of 32 units of 40 chunks (the table path's wider in-kernel merge)."""

import pytest
import torch

import lsh_sampled_sparse_amd as mp
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _layers(cfg, count, **kw):
    out = []
    for layer in range(count):
        inp = synth.config_inputs(cfg, layer=layer, device=DEV, **kw)
        k, v, q = inp["k"], inp["v"], inp["q"].contiguous()
        idx = mp.build_index(k, cfg.K, cfg.L, cfg.hyperplane_seed(layer))
        out.append((k, v, q, idx))
    return out


@pytest.mark.parametrize("tables", [False, True])
def test_repeated_decodes_are_bit_identical(tables):
    cfg = synth.CONFIGS["llama8b_16k"]
    layers = _layers(cfg, 2)
    decode = mp.decode_attn_tables if tables else mp.decode_attn
    if tables:
        for _, _, _, idx in layers:
            mp.build_tables(idx)
    need = max(idx.scratch_bytes(cfg.H_q, tables=tables) for _, _, _, idx in layers)
    scratch = torch.empty(need, dtype=torch.uint8, device=DEV)
    refs = [decode(q, idx, k, v, cfg.n_sink, cfg.n_local, scratch=scratch).clone()
            for k, v, q, idx in layers]
    torch.cuda.synchronize()
    outs = []
    for i in range(200):
        k, v, q, idx = layers[i % 2]
        outs.append(decode(q, idx, k, v, cfg.n_sink, cfg.n_local, scratch=scratch))
    torch.cuda.synchronize()
    bad = [i for i, o in enumerate(outs) if not torch.equal(o, refs[i % 2])]
    assert not bad, f"{len(bad)} of 200 decodes differ from the first, e.g. step {bad[0]}"


def test_repeated_table_decodes_with_the_wide_merge():
    cfg = synth.CONFIGS["batch16_32k"]
    (k, v, q, idx), = _layers(cfg, 1, n=40 * 512, B=4)
    mp.build_tables(idx)
    ref = mp.decode_attn_tables(q, idx, k, v, cfg.n_sink, cfg.n_local).clone()
    torch.cuda.synchronize()
    outs = [mp.decode_attn_tables(q, idx, k, v, cfg.n_sink, cfg.n_local) for _ in range(100)]
    torch.cuda.synchronize()
    bad = [i for i, o in enumerate(outs) if not torch.equal(o, ref)]
    assert not bad, f"{len(bad)} of 100 decodes differ from the first, e.g. step {bad[0]}"
