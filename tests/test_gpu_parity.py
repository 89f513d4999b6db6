"""GPU parity of the HIP path against the fp64 oracle, stage by stage, at sizes
the oracle finishes in seconds (several 512-key chunks and ragged tails), plus
the degenerate cases of the method.  Calls go through the C ABI."""

import math

import numpy as np
import pytest
import torch

import synth
from parity_util import run_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, H_q, H_kv, n, dtype, seed, tail=0.0):
    seeds = [seed + 100 * b for b in range(B)]
    inp = synth.cone_inputs(B=B, H_q=H_q, H_kv=H_kv, n=n, d=128, dtype=dtype, seeds=seeds,
                            tail_frac=tail, device=DEV)
    return inp["k"], inp["v"], inp["q"].contiguous()


def test_tiny_config():
    """The tiny workload exactly: d=128, n=1024, fp32, one head, K=4, L=16,
    T = {0} u last 16, seed 0."""
    cfg = synth.CONFIGS["tiny"]
    inp = synth.config_inputs(cfg, device=DEV)
    r = run_case(inp["k"], inp["v"], inp["q"].contiguous(), cfg.K, cfg.L, cfg.seed, cfg.n_sink,
                 cfg.n_local, name="tiny")
    print("tiny:", r, flush=True)
    assert r["mean_S"] > 100


@pytest.mark.parametrize("name,B,H_q,H_kv,n,dtype,K,L,n_sink,n_local,tail", [
    ("gqa4_bf16_ragged", 1, 8, 2, 1673, torch.bfloat16, 10, 150, 4, 64, 0.0),
    ("batch2_gqa8_tail", 2, 16, 2, 1100, torch.bfloat16, 9, 120, 4, 64, 0.1),
    ("gqa2_fp32", 1, 4, 2, 700, torch.float32, 8, 60, 4, 64, 0.0),
    ("gqa1_bf16_three_chunks", 1, 3, 3, 1536, torch.bfloat16, 6, 40, 2, 32, 0.0),
    ("no_exact_set", 1, 4, 1, 900, torch.bfloat16, 5, 30, 0, 0, 0.0),
    ("all_exact", 1, 4, 1, 300, torch.bfloat16, 5, 30, 100, 250, 0.0),
    ("n_is_5", 1, 4, 1, 5, torch.bfloat16, 4, 16, 1, 1, 0.0),
    ("n_is_1", 1, 2, 1, 1, torch.float32, 4, 16, 0, 0, 0.0),
    ("K16_L255_max", 1, 4, 1, 600, torch.bfloat16, 16, 255, 4, 16, 0.0),
    ("K1_L2_min", 1, 4, 1, 520, torch.bfloat16, 1, 2, 4, 16, 0.0),
    ("two_level_merge_ragged_group", 1, 8, 2, 17 * 512 + 100, torch.bfloat16, 8, 40, 4, 64, 0.0),
    ("three_groups_exact_group_edge", 1, 4, 1, 32 * 512 + 1, torch.bfloat16, 8, 40, 4, 64, 0.0),
])
def test_small_cases(name, B, H_q, H_kv, n, dtype, K, L, n_sink, n_local, tail):
    print(f"case {name}", flush=True)
    k, v, q = _inputs(B, H_q, H_kv, n, dtype, seed=11 + n, tail=tail)
    r = run_case(k, v, q, K, L, seed=5 + K, n_sink=n_sink, n_local=n_local, name=name)
    print(name, r, flush=True)


def test_K0_is_exact_attention():
    """K = 0: every key collides in all L tables and u = 1, so the estimate is
    exact softmax attention over all keys."""
    k, v, q = _inputs(1, 8, 2, 1300, torch.bfloat16, seed=3)
    r = run_case(k, v, q, 0, 8, seed=1, n_sink=4, n_local=64, name="K0_exact")
    import lsh_sampled_sparse_amd as mp
    idx = mp.build_index(k, 0, 8, 1)
    out = mp.decode_attn(q, idx, k, v, 4, 64)
    kf, vf = k.float().cpu(), v.float().cpu()
    qf = q.cpu()
    for hq in range(8):
        h = hq // 4
        w = torch.softmax(kf[0, h].double() @ qf[0, hq].double() / math.sqrt(128), dim=0)
        ref = w @ vf[0, h].double()
        err = (out[0, hq].cpu().double() - ref).abs().max() / ref.abs().max()
        assert err <= 2e-3
    assert r["mean_S"] == 1300 - 68


def test_strided_views():
    """K/V given as a permuted view of a [B][n][H][d] buffer."""
    B, H_q, H_kv, n = 1, 8, 2, 1200
    k, v, q = _inputs(B, H_q, H_kv, n, torch.bfloat16, seed=21)
    k_s = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v_s = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert k_s.stride(1) == 128 and not k_s.is_contiguous()
    r = run_case(k_s, v_s, q, 10, 150, seed=4, n_sink=4, n_local=64, name="strided")
    print("strided", r, flush=True)


def test_explicit_scale():
    k, v, q = _inputs(1, 4, 1, 800, torch.bfloat16, seed=31)
    run_case(k, v, q, 8, 40, seed=2, n_sink=4, n_local=64, scale=0.05)


def test_deterministic():
    import lsh_sampled_sparse_amd as mp
    k, v, q = _inputs(1, 8, 2, 5000, torch.bfloat16, seed=41)
    a = mp.decode_debug(q, mp.build_index(k, 10, 150, 9), k, v, 4, 64)
    b = mp.decode_debug(q, mp.build_index(k, 10, 150, 9), k, v, 4, 64)
    torch.cuda.synchronize()
    assert torch.equal(a["out"], b["out"])
    assert torch.equal(a["s_len"], b["s_len"])
    for hq in range(8):
        m = int(a["s_len"][0, hq])
        assert torch.equal(a["s_idx"][0, hq, :m], b["s_idx"][0, hq, :m])


def test_rejects_mismatched_caches():
    import lsh_sampled_sparse_amd as mp
    k, v, q = _inputs(1, 8, 2, 600, torch.bfloat16, seed=51)
    idx = mp.build_index(k, 10, 150, 9)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):
        mp.decode_attn(q, idx, k[:, :, :500], v[:, :, :500], 4, 64)
    with pytest.raises(mp.MPError, match="MP_E_DTYPE"):
        mp.decode_attn(q, idx, k.float(), v.float(), 4, 64)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):
        mp.decode_attn(q[:, :6].contiguous(), idx, k, v, 4, 64)     # G = 3
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(mp.MPError, match="MP_E_WORKSPACE"):
        mp.decode_attn(q, idx, k, v, 4, 64, scratch=small)


def test_runs_of_two_chunks_every_head():
    """8 KV heads x 98 chunks = 784 chunks, more than the 512 workgroups of the
    grid (256 CUs, 2 a CU up to G = 4): workgroups take runs of two chunks (the gather of
    one chunk after the next one's scan), and with runs aligned to the KV
    heads each head's last run goes to the first workgroups.  Every key's codes;
    counts, sets and outputs on every query head."""
    n = 98 * 512 - 37
    k, v, q = _inputs(1, 32, 8, n, torch.bfloat16, seed=71)
    r = run_case(k, v, q, 8, 40, seed=8, n_sink=4, n_local=64, name="runs_of_two")
    print("runs of two", r, flush=True)


def test_runs_crossing_kv_heads_every_head():
    """8 KV heads x 97 chunks = 776 chunks: runs of two in order, so some runs
    start in one KV head's chunks and end in the next one's.  The next head's
    queries are staged mid-run while the previous head's chunk is still to be
    gathered (the two staging slots), and a head's last chunk (the exact local
    window, a list of more than one round) is gathered inside the run."""
    n = 97 * 512 - 100
    k, v, q = _inputs(1, 32, 8, n, torch.bfloat16, seed=73)
    r = run_case(k, v, q, 8, 40, seed=9, n_sink=4, n_local=64, name="runs_crossing_heads")
    print("runs crossing heads", r, flush=True)


def test_forty_thousand_keys():
    """n = 40,000 (79 chunks, 5 merge groups) at K=10, L=150: every key's
    codes, counts/sets/outputs on all heads."""
    k, v, q = _inputs(1, 8, 2, 40000, torch.bfloat16, seed=61)
    r = run_case(k, v, q, 10, 150, seed=6, n_sink=4, n_local=64, name="40k")
    print("40k", r, flush=True)


def test_zero_query_heads():
    """Two query heads exactly 0 (page "MagicPIG: don't pick the tallest",
    section 5: zero-length vectors need a rule).  Every projection of a zero
    query is 0, so its code is 0 in every table, and each sampled key gets
    cosine 0, p = 1/2.  Small K makes many keys collide with it."""
    import lsh_sampled_sparse_amd as mp
    k, v, q = _inputs(1, 8, 2, 1700, torch.bfloat16, seed=81)
    q[0, 1].zero_()
    q[0, 6].zero_()
    r = run_case(k, v, q, 2, 12, seed=3, n_sink=4, n_local=64, name="zero_query")
    res = mp.decode_debug(q, mp.build_index(k, 2, 12, 3), k, v, 4, 64)
    torch.cuda.synchronize()
    for hq in (1, 6):
        assert not res["qcodes"][0, hq].any()
        assert int(res["s_len"][0, hq]) > 100
    print("zero query", r, flush=True)


def _mirrored_keys(rng, n_pairs, n_center, H_kv):
    """[1][H_kv][2 n_pairs + n_center][128] bf16 keys: pairs c +- delta around
    c in {-1, +1}^128 with delta a multiple of 2^-7 inside (-1, 1), so every
    value is exact in bf16 and the fp64 sums are exact; the mean is c exactly
    in fp64 and fp32, and the n_center keys equal to c center to 0.  Returns
    the keys (positions shuffled, the centers kept outside T) and the center
    positions."""
    n = 2 * n_pairs + n_center
    out = np.empty((1, H_kv, n, 128), dtype=np.float32)
    pos = None
    for h in range(H_kv):
        c = rng.choice([-1.0, 1.0], size=128)
        dlt = np.round(rng.uniform(-0.99, 0.99, size=(n_pairs, 128)) * 128) / 128
        ks = np.concatenate([c + dlt, c - dlt])
        ks = ks[rng.permutation(len(ks))]
        if pos is None:
            pos = np.sort(rng.choice(np.arange(10, n - 100), n_center, replace=False))
        keep = np.ones(n, bool)
        keep[pos] = False
        out[0, h, keep] = ks
        out[0, h, pos] = c
    t = torch.from_numpy(out)
    assert torch.equal(t.to(torch.bfloat16).float(), t)
    return t.to(torch.bfloat16), pos


def test_keys_equal_to_their_mean():
    """Keys equal to their unit's mean (mirrored pairs around an exactly
    representable point): their centered vector is exactly 0 on both sides, so
    their code is 0 in every table and, once sampled, their cosine is 0
    (p = 1/2).  K = 2 makes them collide with most queries."""
    import lsh_sampled_sparse_amd as mp
    rng = np.random.default_rng(91)
    k, pos = _mirrored_keys(rng, 900, 3, 2)
    k = k.to(DEV)
    v = torch.randn(k.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    q = torch.randn(1, 8, 128, generator=torch.Generator().manual_seed(6)).to(DEV) * 0.3
    r = run_case(k, v, q, 2, 16, seed=12, n_sink=4, n_local=64, name="key_equal_to_mean")
    idx = mp.build_index(k, 2, 16, 12)
    res = mp.decode_debug(q, idx, k, v, 4, 64)
    torch.cuda.synchronize()
    _, mu, _ = idx.views()
    for h in range(2):
        assert torch.equal(mu[0, h].cpu(), k[0, h, pos[0]].float().cpu())
    sampled = 0
    for hq in range(8):
        m = int(res["s_len"][0, hq])
        sampled += int(np.isin(pos, res["s_idx"][0, hq, :m].cpu().numpy()).sum())
    assert sampled >= 12, sampled          # of 24 (key, head) pairs; u(1/2) = 0.94 here
    print("key equal to mean", r, "sampled centers:", sampled, flush=True)
