"""GPU parity of the incremental index (mp_build_index_cap, mp_index_append),
through the C ABI.

An index is built over the first n0 keys of a key cache with room for more,
then grown step by step to longer prefixes of the same cache.  The reading
checked (the pages do not say how the mean moves as keys arrive): appended
keys are centered by the mean of the n0 keys the index was built on, and
encoded with the same hyperplanes.  After every append:
  * mu is bit for bit the one of the build;
  * every key's codes (old and appended) match the oracle's encoding of
    k - mu0 outside the 1e-5 band, with mismatches under 0.01% of bits;
  * counts and sampled sets are exact (the oracle's integer steps on the
    GPU's codes), with T taken at the new length;
  * outputs are within 2e-3 per row of the oracle's fp64 estimator with mu0;
  * mp_decode_attn equals mp_decode_debug bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import lsh_sampled_sparse_amd as mp
import oracle
import synth
from parity_util import (OUT_TOL, check_codes, check_unit_codes, gpu_codes_table_major,
                         oracle_threads, row_rel_err)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cache(B, H_q, H_kv, n, dtype, seed):
    seeds = [seed + 100 * b for b in range(B)]
    inp = synth.cone_inputs(B=B, H_q=H_q, H_kv=H_kv, n=n, d=128, dtype=dtype, seeds=seeds,
                            device=DEV)
    return inp["k"], inp["v"], inp["q"].contiguous()


def check_index(idx, k, v, q, n, n0, K, L, seed, n_sink, n_local):
    B, H_kv = k.shape[:2]
    H_q = q.shape[1]
    G = H_q // H_kv
    kk, vv = k[:, :, :n], v[:, :, :n]
    res = mp.decode_debug(q, idx, kk, vv, n_sink, n_local)
    out2 = mp.decode_attn(q, idx, kk, vv, n_sink, n_local)
    torch.cuda.synchronize()
    assert torch.equal(res["out"], out2), "mp_decode_attn and mp_decode_debug differ"
    W = oracle.hyperplanes(seed, K * L, 128)
    codes = gpu_codes_table_major(idx)
    assert codes.shape[-1] == n
    qcodes = res["qcodes"].cpu().numpy().view(np.uint16)
    counts = res["counts"].cpu().numpy().astype(np.int32)
    s_idx = res["s_idx"].cpu().numpy()
    s_len = res["s_len"].cpu().numpy()
    out = res["out"].cpu().double().numpy()
    scl = 1.0 / math.sqrt(128)
    errs, mism, bits = [], 0, 0
    for b in range(B):
        for h in range(H_kv):
            kh = k[b, h, :n].cpu().double().numpy()
            vh = v[b, h, :n].cpu().double().numpy()
            mu0 = oracle.mean(k[b, h, :n0].cpu().double().numpy())     # frozen at build
            ref, band, _ = oracle.encode_keys_band_parallel(kh, W, K, L, mu0, oracle_threads())
            m_, _ = check_unit_codes(ref, band, codes[b, h], f"key codes ({b},{h}), n={n}")
            mism += m_
            bits += n * K * L
            for g in range(G):
                hq = h * G + g
                qh = q[b, hq].cpu().double().numpy()
                check_codes(qh[None], W, K, L, qcodes[b, hq][None], "query")
                cnt = oracle.collision_counts(codes[b, h], qcodes[b, hq])
                assert np.array_equal(cnt, counts[b, hq]), f"counts differ at ({b},{hq}), n={n}"
                S = oracle.select(cnt, n_sink, n_local)
                assert s_len[b, hq] == len(S) and np.array_equal(S, s_idx[b, hq, :len(S)]), \
                    f"S differs at ({b},{hq}), n={n}"
                ref = oracle.estimate(qh, kh, vh, mu0, S, K, L, n_sink, n_local, scl)
                e = row_rel_err(out[b, hq], ref)
                errs.append(e)
                assert e <= OUT_TOL, f"output error {e:.3g} at ({b},{hq}), n={n}"
    return dict(n=n, max_out_err=max(errs) if errs else 0.0, mismatched_bits=mism, bits=bits,
                mean_S=float(s_len.mean()))


def run_growth(B, H_q, H_kv, dtype, K, L, n0, steps, n_sink, n_local, seed, **kw):
    cap = max(steps + [n0])
    k, v, q = _cache(B, H_q, H_kv, cap, dtype, seed)
    idx = mp.build_index(k[:, :, :n0], K, L, seed, capacity=cap)
    torch.cuda.synchronize()
    mu_built = idx.views()[1].clone()
    reps = [check_index(idx, k, v, q, n0, n0, K, L, seed, n_sink, n_local, **kw)]
    for n in steps:
        mp.append_index(idx, k[:, :, :n])
        torch.cuda.synchronize()
        assert idx.n == n
        assert torch.equal(idx.views()[1], mu_built), "mu moved on append"
        reps.append(check_index(idx, k, v, q, n, n0, K, L, seed, n_sink, n_local, **kw))
    return reps


def test_grow_bf16_gqa4_across_words_blocks_and_chunks():
    # 700 -> 701 (inside a word), 1023, 1024 (block edge), 1500, 2600 (new chunks)
    for r in run_growth(1, 8, 2, torch.bfloat16, 10, 60, 700, [701, 1023, 1024, 1500, 2600],
                        4, 32, seed=21):
        print("bf16 growth", r, flush=True)


def test_grow_fp32_batch2_gqa2_with_a_no_op_step():
    for r in run_growth(2, 4, 2, torch.float32, 8, 40, 300, [300, 513, 1100], 2, 16, seed=22):
        print("fp32 growth", r, flush=True)


def test_grow_from_one_key_gqa8():
    for r in run_growth(1, 8, 1, torch.bfloat16, 6, 24, 1, [2, 255, 256, 257, 800], 1, 8,
                        seed=23):
        print("from one key", r, flush=True)


@pytest.mark.parametrize("dtype,H_q,K,L", [(torch.bfloat16, 8, 10, 60), (torch.float32, 16, 9, 40)])
def test_small_appends_bit_by_bit(dtype, H_q, K, L):
    """Appends of at most 64 keys write the new keys' bits alone into the
    plane words; 65 or more re-encode from the first new key's 256-key block.
    From 480 keys: steps of 1, 1, 31 (into the second chunk), 32, 64, 65 (the
    block path), 349, 1, 1 (into the third chunk) and 63 keys."""
    for r in run_growth(1, H_q, 2, dtype, K, L, 480,
                        [481, 482, 513, 545, 609, 674, 1023, 1024, 1025, 1088], 4, 32, seed=26):
        print("small appends", r, flush=True)


@pytest.mark.timeout(600)
def test_grow_96k_key_by_key():
    """The serving pattern at the timed shape: one key appended per step
    (a token leaving the local window), three steps."""
    cfg = synth.CONFIGS["llama8b_96k"]
    n1 = cfg.n
    for r in run_growth(1, cfg.H_q, cfg.H_kv, cfg.dtype, cfg.K, cfg.L, n1 - 3,
                        [n1 - 2, n1 - 1, n1], cfg.n_sink, cfg.n_local,
                        seed=cfg.hyperplane_seed(4)):
        print("96k key by key", r, flush=True)


def test_grow_K0_every_key_collides():
    for r in run_growth(1, 4, 1, torch.bfloat16, 0, 8, 200, [900], 4, 16, seed=24):
        print("K0 growth", r, flush=True)


@pytest.mark.timeout(600)
def test_grow_96k_one_layer():
    """The timed workload's shape: built 300 keys short of 96K, grown in two
    steps; every key's codes and every head's counts, set and output after
    each step."""
    cfg = synth.CONFIGS["llama8b_96k"]
    n1 = cfg.n
    for r in run_growth(1, cfg.H_q, cfg.H_kv, cfg.dtype, cfg.K, cfg.L, n1 - 300,
                        [n1 - 211, n1], cfg.n_sink, cfg.n_local, seed=cfg.hyperplane_seed(2)):
        print("96k growth", r, flush=True)


def test_tables_after_append_are_rebuilt_and_agree():
    k, v, q = _cache(1, 8, 2, 3000, torch.bfloat16, 25)
    idx = mp.build_index(k[:, :, :1200], 9, 50, 25, capacity=3000)
    mp.build_tables(idx)
    mp.append_index(idx, k[:, :, :3000])
    assert idx.tables is None
    with pytest.raises(mp.MPError, match="MP_E_ARG"):
        mp.decode_attn_tables(q, idx, k, v, 4, 32)
    mp.build_tables(idx)
    rt = mp.decode_tables_debug(q, idx, k, v, 4, 32)
    rs = mp.decode_debug(q, idx, k, v, 4, 32)
    torch.cuda.synchronize()
    assert torch.equal(rt["s_len"], rs["s_len"])
    assert np.array_equal(rt["counts"].cpu().numpy(), np.minimum(rs["counts"].cpu().numpy(), 2))
    err = max(row_rel_err(a, b) for a, b in zip(rt["out"].cpu().double().numpy().reshape(-1, 128),
                                                rs["out"].cpu().double().numpy().reshape(-1, 128)))
    assert err <= 1e-5, err


def test_append_rejections():
    k, v, q = _cache(1, 4, 1, 1000, torch.bfloat16, 26)
    idx = mp.build_index(k[:, :, :600], 8, 20, 26, capacity=900)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # fewer keys than indexed
        mp.append_index(idx, k[:, :, :599])
    assert idx.n == 600
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # beyond the capacity
        mp.append_index(idx, k[:, :, :901])
    with pytest.raises(mp.MPError, match="MP_E_DTYPE"):
        mp.append_index(idx, k[:, :, :700].float())
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # decode at the old length
        mp.append_index(idx, k[:, :, :700])
        mp.decode_attn(q, idx, k[:, :, :600], v[:, :, :600], 4, 16)
    with pytest.raises(mp.MPError, match="MP_E_ARG"):
        mp.build_index(k[:, :, :600], 8, 20, 26, capacity=599)


def _key_bits_mask(n, nc, device):
    """int32 mask [nc][1][16] of the plane bits that hold keys < n (bit j of
    word w of chunk c is key 512c + 32w + j); the words of a chunk past n
    hold whatever the workspace held."""
    key0 = torch.arange(nc, device=device)[:, None] * 512 + torch.arange(16, device=device) * 32
    nv = (n - key0).clamp(0, 32)
    m = torch.where(nv >= 32, torch.full_like(nv, -1), (1 << nv.clamp(max=31)) - 1)
    return m.to(torch.int32)[:, None, :]


def _twin_steps(B, H_q, H_kv, dtype, K, L, n0, steps, n_sink, n_local, seed, cap=None):
    """Two indexes built alike over the first n0 keys; each step grows one
    with mp_index_append + mp_decode_attn and the other with
    mp_decode_attn_append.  Outputs, n and every key's plane bits must agree
    bit for bit.  Returns the second index and the cache."""
    cap = cap or max(steps + [n0])
    k, v, q = _cache(B, H_q, H_kv, cap, dtype, seed)
    ia = mp.build_index(k[:, :, :n0], K, L, seed, capacity=cap)
    ib = mp.build_index(k[:, :, :n0], K, L, seed, capacity=cap)
    if 0 < K <= 12:
        mp.build_tables(ib)   # detached by the first step
    for n in steps:
        mp.append_index(ia, k[:, :, :n])
        oa = mp.decode_attn(q, ia, k[:, :, :n], v[:, :, :n], n_sink, n_local)
        ob = mp.decode_attn_append(q, ib, k[:, :, :n], v[:, :, :n], n_sink, n_local)
        torch.cuda.synchronize()
        assert ia.n == ib.n == n
        assert ib.tables is None
        assert torch.equal(oa, ob), f"outputs differ at n={n}"
        pa, pb = ia.views()[2], ib.views()[2]
        m = _key_bits_mask(n, pa.shape[2], pa.device)
        assert torch.equal(pa & m, pb & m), f"plane bits of the keys differ at n={n}"
        print(f"n={n}: outputs and the key bits of {pb.numel()} plane words equal", flush=True)
    return ib, k, v, q


@pytest.mark.parametrize("dtype,H_q,H_kv,K,L", [(torch.bfloat16, 8, 2, 10, 60),
                                                (torch.float32, 8, 1, 9, 40)])
def test_decode_attn_append_equals_append_then_decode(dtype, H_q, H_kv, K, L):
    """From 480 keys: 1 key (inside a word), 30, 1 (the chunk's last key), 1
    (into the second chunk), 64 (the most one encode launch appends), 65
    (the two-call route), no new key, 1, and 63 keys; then the grown index
    against the oracle."""
    steps = [481, 511, 512, 513, 577, 642, 642, 643, 706]
    ib, k, v, q = _twin_steps(1, H_q, H_kv, dtype, K, L, 480, steps, 4, 32, seed=27, cap=1100)
    r = check_index(ib, k, v, q, 706, 480, K, L, 27, 4, 32)
    print("fused append, oracle", r, flush=True)


def test_decode_attn_append_batch2_and_K0():
    _twin_steps(2, 8, 2, torch.bfloat16, 8, 30, 1000, [1001, 1040, 1600], 4, 16, seed=28)
    _twin_steps(1, 4, 1, torch.bfloat16, 0, 8, 200, [201, 230], 4, 16, seed=29)


@pytest.mark.parametrize("n_local,steps", [(0, [701, 702, 703]), (4, [701, 709, 710]),
                                           (64, [701, 702, 717, 733])])
def test_decode_attn_append_with_and_without_a_local_window(n_local, steps):
    """The appended keys' codes must be in the planes before the scan reads
    them whether or not the new keys are in the exact set T.  From 700 keys:
    with no local window (every new key is sampled or not by its codes),
    with 4 local keys (1, then 8 new keys: some outside T), and with 64 (1,
    1, 15 and 16 new keys, all in T)."""
    ib, k, v, q = _twin_steps(1, 8, 2, torch.bfloat16, 10, 60, 700, steps, 4, n_local, seed=31,
                              cap=800)
    r = check_index(ib, k, v, q, steps[-1], 700, 10, 60, 31, 4, n_local)
    print("append with n_local", n_local, r, flush=True)


def test_decode_attn_append_rejections_leave_the_index():
    k, v, q = _cache(1, 4, 1, 1000, torch.bfloat16, 30)
    idx = mp.build_index(k[:, :, :600], 8, 20, 30, capacity=900)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # beyond the capacity
        mp.decode_attn_append(q, idx, k[:, :, :901], v[:, :, :901], 4, 16)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # v at another length
        mp.decode_attn_append(q, idx, k[:, :, :610], v[:, :, :600], 4, 16)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):        # v at another length, many keys
        mp.decode_attn_append(q, idx, k[:, :, :800], v[:, :, :600], 4, 16)
    assert idx.n == 600
    mp.decode_attn(q, idx, k[:, :, :600], v[:, :, :600], 4, 16)   # still 600 keys
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_decode_attn_append_96k_key_by_key():
    """The serving pattern at the timed shape: one key appended per decode
    step, through the fused call and through the two calls."""
    cfg = synth.CONFIGS["llama8b_96k"]
    n1 = cfg.n
    _twin_steps(1, cfg.H_q, cfg.H_kv, cfg.dtype, cfg.K, cfg.L, n1 - 4, [n1 - 3, n1 - 2, n1 - 1, n1],
                cfg.n_sink, cfg.n_local, seed=cfg.hyperplane_seed(5))
