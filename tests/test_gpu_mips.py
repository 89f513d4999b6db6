"""GPU parity of the inner-product-to-cosine lift (MP_INDEX_MIPS), through the
C ABI (page "MagicPIG: LSH Sampling for Efficient LLM Generation", method
details: keys lifted to [x, sqrt(r^2 - |x|^2)], queries to [q, 0]; here x is
the centered key).

Checked on every case:
  * W and the extra hyperplane coordinate within one fp32 ulp of the oracle's;
  * the radius r of every unit within 2e-6 of the oracle's fp64 r;
  * key codes against the oracle's codes of the lifted keys under the lifted
    hyperplanes, exact outside the 1e-5 band (taken on the lifted pair), with
    mismatches under 0.01% of bits;
  * query codes, counts and sampled sets exact (oracle integer steps on the
    GPU's codes);
  * outputs within 2e-3 per row of the oracle's estimator with the lifted
    cosine q.x / (|q| r);
  * mp_decode_attn equals mp_decode_debug bit for bit.
The 256K workload also compares the estimator error of the plain and the
lifted index against exact attention (reported, not asserted either way: the
pages give no figure for it).
"""

import math

import numpy as np
import pytest
import torch

import lsh_sampled_sparse_amd as mp
import oracle
import synth
from parity_util import (OUT_TOL, check_codes, check_unit_codes, gpu_codes_table_major,
                         oracle_threads, row_rel_err, ulp_distance_f32)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, H_q, H_kv, n, dtype, seed, tail=0.0):
    seeds = [seed + 100 * b for b in range(B)]
    inp = synth.cone_inputs(B=B, H_q=H_q, H_kv=H_kv, n=n, d=128, dtype=dtype, seeds=seeds,
                            tail_frac=tail, device=DEV)
    return inp["k"], inp["v"], inp["q"].contiguous()


def run_lifted_case(k, v, q, K, L, seed, n_sink, n_local):
    B, H_kv, n, d = k.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    idx = mp.build_index(k, K, L, seed, mips=True)
    res = mp.decode_debug(q, idx, k, v, n_sink, n_local)
    out2 = mp.decode_attn(q, idx, k, v, n_sink, n_local)
    torch.cuda.synchronize()
    assert torch.equal(res["out"], out2), "mp_decode_attn and mp_decode_debug differ"
    W_gpu, mu_gpu, _ = idx.views()
    wx_gpu, r_gpu = (t.cpu().numpy() for t in idx.lift_views())
    R = K * L
    W = oracle.hyperplanes(seed, R, d)
    w = oracle.hyperplane_extra(seed, R, d)
    assert ulp_distance_f32(W, W_gpu.cpu().numpy()).max(initial=0) <= 1
    assert ulp_distance_f32(w, wx_gpu).max(initial=0) <= 1
    Wl = np.concatenate([W, w[:, None]], axis=1).astype(np.float32)     # lifted hyperplanes
    codes = gpu_codes_table_major(idx)
    qcodes = res["qcodes"].cpu().numpy().view(np.uint16)
    counts = res["counts"].cpu().numpy().astype(np.int32)
    s_idx = res["s_idx"].cpu().numpy()
    s_len = res["s_len"].cpu().numpy()
    out = res["out"].cpu().double().numpy()
    scl = 1.0 / math.sqrt(d)
    errs, mism, bits = [], 0, 0
    for b in range(B):
        for h in range(H_kv):
            kh = k[b, h].cpu().double().numpy()
            vh = v[b, h].cpu().double().numpy()
            mu = oracle.mean(kh)
            r = oracle.aug_radius(kh, mu)
            assert abs(float(r_gpu[b, h]) - r) <= 2e-6 * r, (float(r_gpu[b, h]), r)
            x = kh - mu
            lift = np.sqrt(np.maximum(r * r - (x * x).sum(axis=1), 0.0))
            xl = np.concatenate([x, lift[:, None]], axis=1)
            if K > 0:
                # the lifted keys against the lifted hyperplanes, band taken on the lifted pair
                ref, band, _ = oracle.encode_keys_band_parallel(xl, Wl, K, L, None,
                                                                oracle_threads())
                m_, _ = check_unit_codes(ref, band, codes[b, h], f"lifted key codes ({b},{h})")
                mism += m_
                bits += n * K * L
            for g in range(G):
                hq = h * G + g
                qh = q[b, hq].cpu().double().numpy()
                if K > 0:
                    check_codes(qh[None], W, K, L, qcodes[b, hq][None], "query")
                cnt = oracle.collision_counts(codes[b, h], qcodes[b, hq])
                assert np.array_equal(cnt, counts[b, hq]), f"counts differ at ({b},{hq})"
                S = oracle.select(cnt, n_sink, n_local)
                assert s_len[b, hq] == len(S) and np.array_equal(S, s_idx[b, hq, :len(S)]), \
                    f"S differs at ({b},{hq})"
                ref = oracle.estimate(qh, kh, vh, mu, S, K, L, n_sink, n_local, scl, aug_r=r)
                e = row_rel_err(out[b, hq], ref)
                errs.append(e)
                assert e <= OUT_TOL, f"output error {e:.3g} at ({b},{hq})"
    rep = dict(max_out_err=max(errs) if errs else 0.0, mismatched_bits=mism, bits=bits,
               mean_S=float(s_len.mean()))
    return idx, rep


@pytest.mark.parametrize("name,B,H_q,H_kv,n,dtype,K,L,n_sink,n_local,tail", [
    ("gqa4_bf16_ragged", 1, 8, 2, 1673, torch.bfloat16, 10, 150, 4, 64, 0.0),
    ("batch2_gqa2_fp32_tail", 2, 4, 2, 1100, torch.float32, 8, 60, 4, 32, 0.1),
    ("gqa8_bf16", 1, 16, 2, 2100, torch.bfloat16, 9, 120, 4, 64, 0.0),
    ("gqa1_three_chunks", 1, 3, 3, 1536, torch.bfloat16, 6, 40, 2, 32, 0.0),
    ("n_is_5", 1, 4, 1, 5, torch.bfloat16, 4, 16, 1, 1, 0.0),
    ("K0_every_key", 1, 4, 1, 700, torch.bfloat16, 0, 8, 4, 16, 0.0),
    ("K16_L255_max", 1, 4, 1, 600, torch.bfloat16, 16, 255, 4, 16, 0.0),
])
def test_small_cases(name, B, H_q, H_kv, n, dtype, K, L, n_sink, n_local, tail):
    print(f"case {name}", flush=True)
    k, v, q = _inputs(B, H_q, H_kv, n, dtype, seed=31 + n, tail=tail)
    _, r = run_lifted_case(k, v, q, K, L, seed=9 + K, n_sink=n_sink, n_local=n_local)
    print(name, r, flush=True)


def test_tables_on_a_lifted_index_agree_with_its_scan():
    k, v, q = _inputs(1, 8, 2, 5000, torch.bfloat16, seed=33)
    idx, _ = run_lifted_case(k, v, q, 10, 150, seed=33, n_sink=4, n_local=64)
    mp.build_tables(idx)
    rt = mp.decode_tables_debug(q, idx, k, v, 4, 64)
    rs = mp.decode_debug(q, idx, k, v, 4, 64)
    torch.cuda.synchronize()
    assert torch.equal(rt["s_len"], rs["s_len"])
    assert np.array_equal(rt["counts"].cpu().numpy(), np.minimum(rs["counts"].cpu().numpy(), 2))
    err = max(row_rel_err(a, b) for a, b in zip(rt["out"].cpu().double().numpy().reshape(-1, 128),
                                                rs["out"].cpu().double().numpy().reshape(-1, 128)))
    assert err <= 1e-5, err


def test_lifted_index_refuses_to_grow_and_plain_views():
    k, v, q = _inputs(1, 4, 1, 900, torch.bfloat16, seed=34)
    idx = mp.build_index(k[:, :, :600], 8, 20, 34, mips=True, capacity=900)
    with pytest.raises(mp.MPError, match="MP_E_ARG"):
        mp.append_index(idx, k[:, :, :700])
    plain = mp.build_index(k, 8, 20, 34)
    with pytest.raises(mp.MPError, match="MP_E_ARG"):
        plain.lift_views()


@pytest.mark.timeout(600)
def test_llama8b_96k_lifted():
    """The timed workload with the lift: every key's lifted codes, every
    head's counts, set and output."""
    cfg = synth.CONFIGS["llama8b_96k"]
    inp = synth.config_inputs(cfg, layer=3, device=DEV)
    _, r = run_lifted_case(inp["k"], inp["v"], inp["q"].contiguous(), cfg.K, cfg.L,
                           cfg.hyperplane_seed(3), cfg.n_sink, cfg.n_local)
    print("llama8b_96k lifted", r, flush=True)


def test_llama70b_256k_plain_vs_lifted_estimator_error():
    """Mean over query heads of |o_hat - o| / |o| against exact attention
    (plain PyTorch fp32), for the plain and the lifted index at L = 60, 120,
    240; both must fall as L grows."""
    cfg = synth.CONFIGS["llama70b_256k"]
    inp = synth.config_inputs(cfg, device=DEV)
    k, v, q = inp["k"], inp["v"], inp["q"].contiguous()
    G = cfg.H_q // cfg.H_kv
    ref = torch.empty(cfg.H_q, cfg.d, device=DEV)
    for h in range(cfg.H_kv):
        kf, vf = k[0, h].float(), v[0, h].float()
        for g in range(G):
            w = torch.softmax(kf @ q[0, h * G + g] / math.sqrt(cfg.d), dim=0)
            ref[h * G + g] = w @ vf
    errs = {}
    for mips in (False, True):
        for L in cfg.l_sweep:
            idx = mp.build_index(k, cfg.K, L, cfg.hyperplane_seed(0), mips=mips)
            res = mp.decode_debug(q, idx, k, v, cfg.n_sink, cfg.n_local)
            torch.cuda.synchronize()
            e = ((res["out"][0] - ref).norm(dim=-1) / ref.norm(dim=-1)).mean().item()
            errs[("lifted" if mips else "plain", L)] = (round(e, 5),
                                                         round(float(res["s_len"].float().mean()), 1))
            del idx, res
    print("estimator error, mean |S| per head (256K, K=9):", errs, flush=True)
    Ls = list(cfg.l_sweep)
    for kind in ("plain", "lifted"):
        for a, b in zip(Ls, Ls[1:]):
            assert errs[(kind, b)][0] < errs[(kind, a)][0], (kind, errs)
