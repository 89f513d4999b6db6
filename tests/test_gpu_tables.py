"""GPU parity of the bucketed-table decode path (mp_build_tables,
mp_decode_attn_tables / mp_decode_tables_debug), through the C ABI.

Checked on every case:
  * the tables themselves, exactly: per (unit, table) the bucket starts run
    from 0 to n without decreasing, the entries are a permutation of the keys,
    and every key sits in the bucket of its own code (the GPU's codes);
  * min(count, 2) per key and head, and the sampled sets, exactly against
    the oracle's integer steps on the GPU's codes and against the code-scan
    path (both must find the same set: the method defines it, not the route);
  * outputs within 2e-3 per row of the oracle's fp64 estimator on that set,
    and equal to the code-scan path's up to fp32 rounding;
  * mp_decode_attn_tables equals mp_decode_tables_debug bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import lsh_sampled_sparse_amd as mp
import oracle
import synth
from parity_util import OUT_TOL, gpu_codes_table_major, row_rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, H_q, H_kv, n, dtype, seed, tail=0.0):
    seeds = [seed + 100 * b for b in range(B)]
    inp = synth.cone_inputs(B=B, H_q=H_q, H_kv=H_kv, n=n, d=128, dtype=dtype, seeds=seeds,
                            tail_frac=tail, device=DEV)
    return inp["k"], inp["v"], inp["q"].contiguous()


def check_tables(idx, codes, units=None, tables=None):
    """Exact structure of the tables against the GPU's codes [B][H][L][n]."""
    offs, ents = idx.table_views()
    offs = offs.cpu().numpy().view(np.uint32)
    ents = ents.cpu().numpy().view(np.uint32)
    B, H, L, n = codes.shape
    nb = 1 << idx.K
    for b in range(B):
        for h in range(H):
            if units is not None and (b, h) not in units:
                continue
            for l in (range(L) if tables is None else tables):
                o = offs[b, h, l].astype(np.int64)
                assert o[0] == 0 and o[nb] == n, "bucket starts do not span [0, n]"
                sizes = np.diff(o)
                assert (sizes >= 0).all(), "bucket starts decrease"
                e = ents[b, h, l].astype(np.int64)
                assert np.array_equal(np.sort(e), np.arange(n)), "entries are not the keys"
                want = np.repeat(np.arange(nb), sizes)
                assert np.array_equal(codes[b, h, l][e], want), "a key sits in another bucket"


def run_tables_case(k, v, q, K, L, seed, n_sink, n_local, scale=0.0, heads=None,
                    table_units=None, table_rows=None):
    B, H_kv, n, d = k.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    idx = mp.build_index(k, K, L, seed)
    mp.build_tables(idx)
    rt = mp.decode_tables_debug(q, idx, k, v, n_sink, n_local, scale=scale)
    out_t = mp.decode_attn_tables(q, idx, k, v, n_sink, n_local, scale=scale)
    rs = mp.decode_debug(q, idx, k, v, n_sink, n_local, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(rt["out"], out_t), "tables: production and debug outputs differ"
    codes = gpu_codes_table_major(idx)
    check_tables(idx, codes, units=table_units, tables=table_rows)

    c2 = rt["counts"].cpu().numpy().astype(np.int32)
    cs = rs["counts"].cpu().numpy().astype(np.int32)
    assert np.array_equal(c2, np.minimum(cs, 2)), "min(count, 2) differs from the code scan"
    assert torch.equal(rt["s_len"], rs["s_len"]), "|S| differs from the code scan"
    assert torch.equal(rt["qcodes"], rs["qcodes"])
    s_len = rt["s_len"].cpu().numpy()
    s_t = rt["s_idx"].cpu().numpy()
    s_s = rs["s_idx"].cpu().numpy()
    out = rt["out"].cpu().double().numpy()
    out_s = rs["out"].cpu().double().numpy()
    qc = rt["qcodes"].cpu().numpy().view(np.uint16)
    W_gpu, mu_gpu, _ = idx.views()
    scl = scale if scale > 0 else 1.0 / math.sqrt(d)
    errs, diffs = [], []
    for b in range(B):
        for h in range(H_kv):
            kh = vh = mu = None
            for g in range(G):
                hq = h * G + g
                m = int(s_len[b, hq])
                assert np.array_equal(s_t[b, hq, :m], s_s[b, hq, :m]), f"S differs at ({b},{hq})"
                diffs.append(row_rel_err(out[b, hq], out_s[b, hq]))
                if heads is not None and (b, hq) not in heads:
                    continue
                if kh is None:
                    kh = k[b, h].cpu().double().numpy()
                    vh = v[b, h].cpu().double().numpy()
                    mu = oracle.mean(kh)
                cnt = oracle.collision_counts(codes[b, h], qc[b, hq])
                assert np.array_equal(np.minimum(cnt, 2), c2[b, hq]), f"counts at ({b},{hq})"
                S = oracle.select(cnt, n_sink, n_local)
                assert m == len(S) and np.array_equal(S, s_t[b, hq, :m]), f"S vs oracle ({b},{hq})"
                qh = q[b, hq].cpu().double().numpy()
                ref = oracle.estimate(qh, kh, vh, mu, S, K, L, n_sink, n_local, scl)
                e = row_rel_err(out[b, hq], ref)
                errs.append(e)
                assert e <= OUT_TOL, f"output error {e:.3g} at ({b},{hq})"
    assert max(diffs) <= 1e-5, f"tables and code scan outputs differ by {max(diffs):.3g}"
    rep = dict(max_out_err=max(errs) if errs else 0.0, max_vs_scan=max(diffs),
               mean_S=float(s_len.mean()))
    del idx
    return rep


def test_tiny_config():
    cfg = synth.CONFIGS["tiny"]
    inp = synth.config_inputs(cfg, device=DEV)
    r = run_tables_case(inp["k"], inp["v"], inp["q"].contiguous(), cfg.K, cfg.L, cfg.seed,
                        cfg.n_sink, cfg.n_local)
    print("tiny tables:", r, flush=True)


@pytest.mark.parametrize("name,B,H_q,H_kv,n,dtype,K,L,n_sink,n_local,tail", [
    ("gqa4_bf16_ragged", 1, 8, 2, 1673, torch.bfloat16, 10, 150, 4, 64, 0.0),
    ("batch2_gqa8_tail", 2, 16, 2, 1100, torch.bfloat16, 9, 120, 4, 64, 0.1),
    ("gqa2_fp32", 1, 4, 2, 700, torch.float32, 8, 60, 4, 64, 0.0),
    ("gqa1_bf16_three_chunks", 1, 3, 3, 1536, torch.bfloat16, 6, 40, 2, 32, 0.0),
    ("no_exact_set", 1, 4, 1, 900, torch.bfloat16, 5, 30, 0, 0, 0.0),
    ("all_exact", 1, 4, 1, 300, torch.bfloat16, 5, 30, 100, 250, 0.0),
    ("n_is_5", 1, 4, 1, 5, torch.bfloat16, 4, 16, 1, 1, 0.0),
    ("n_is_1", 1, 2, 1, 1, torch.float32, 4, 16, 0, 0, 0.0),
    ("K12_L255_max", 1, 4, 1, 600, torch.bfloat16, 12, 255, 4, 16, 0.0),
    ("K1_L2_min", 1, 4, 1, 520, torch.bfloat16, 1, 2, 4, 16, 0.0),
    ("K0_every_key", 1, 8, 2, 1300, torch.bfloat16, 0, 8, 4, 64, 0.0),
    ("two_level_merge_ragged_group", 1, 8, 2, 17 * 512 + 100, torch.bfloat16, 8, 40, 4, 64, 0.0),
    # 32 units of 36 and 40 chunks: table_gather merges a unit's records in
    # the kernel (many units), and the scan its runs' records
    ("merge_in_kernel_32_units", 2, 32, 16, 35 * 512 + 7, torch.bfloat16, 8, 40, 4, 64, 0.0),
    ("merge_in_kernel_32_units_gqa4", 4, 32, 8, 40 * 512 - 3, torch.bfloat16, 8, 40, 4, 64, 0.0),
])
def test_small_cases(name, B, H_q, H_kv, n, dtype, K, L, n_sink, n_local, tail):
    print(f"case {name}", flush=True)
    k, v, q = _inputs(B, H_q, H_kv, n, dtype, seed=11 + n, tail=tail)
    r = run_tables_case(k, v, q, K, L, seed=5 + K, n_sink=n_sink, n_local=n_local)
    print(name, r, flush=True)


def test_forty_thousand_keys():
    k, v, q = _inputs(1, 8, 2, 40000, torch.bfloat16, seed=61)
    r = run_tables_case(k, v, q, 10, 150, seed=6, n_sink=4, n_local=64)
    print("40k tables", r, flush=True)


def test_llama8b_96k_one_layer():
    """The timed workload: every head's set against the code scan and its
    output against the oracle, and the tables of two units in full."""
    cfg = synth.CONFIGS["llama8b_96k"]
    inp = synth.config_inputs(cfg, layer=5, device=DEV)
    r = run_tables_case(inp["k"], inp["v"], inp["q"].contiguous(), cfg.K, cfg.L,
                        cfg.hyperplane_seed(5), cfg.n_sink, cfg.n_local,
                        table_units=[(0, 0), (0, 7)])
    print("llama8b_96k tables", r, flush=True)


@pytest.mark.timeout(600)
def test_batch16_32k_tables_against_the_scan():
    """The batch-16 workload (128 units of 64 chunks, whose records the
    table path merges inside table_gather): every head's sampled set and
    counts capped at 2 equal the code scan's, outputs within 1e-5 of it
    (the two paths fold the same rows in another order)."""
    cfg = synth.CONFIGS["batch16_32k"]
    inp = synth.config_inputs(cfg, device=DEV)
    k, v, q = inp["k"], inp["v"], inp["q"].contiguous()
    idx = mp.build_index(k, cfg.K, cfg.L, cfg.hyperplane_seed(0))
    mp.build_tables(idx)
    rt = mp.decode_tables_debug(q, idx, k, v, cfg.n_sink, cfg.n_local)
    rs = mp.decode_debug(q, idx, k, v, cfg.n_sink, cfg.n_local)
    ot = mp.decode_attn_tables(q, idx, k, v, cfg.n_sink, cfg.n_local)
    torch.cuda.synchronize()
    assert torch.equal(rt["out"], ot), "debug and production table decodes differ"
    assert torch.equal(rt["s_len"], rs["s_len"])
    assert torch.equal(rt["counts"], torch.minimum(rs["counts"], torch.full_like(rs["counts"], 2)))
    err = max(row_rel_err(a, b)
              for a, b in zip(rt["out"].cpu().double().numpy().reshape(-1, 128),
                              rs["out"].cpu().double().numpy().reshape(-1, 128)))
    print("batch16 tables vs scan", err, flush=True)
    assert err <= 1e-5, err


@pytest.mark.timeout(600)
def test_llama70b_256k_every_head():
    """The 256K workload (G = 8): every head's set against the code scan and
    its output against the oracle; the tables of one unit, three of them in
    full."""
    cfg = synth.CONFIGS["llama70b_256k"]
    inp = synth.config_inputs(cfg, device=DEV)
    r = run_tables_case(inp["k"], inp["v"], inp["q"].contiguous(), cfg.K, cfg.L,
                        cfg.hyperplane_seed(0), cfg.n_sink, cfg.n_local,
                        table_units=[(0, 3)], table_rows=[0, 59, 119])
    print("llama70b_256k tables", r, flush=True)


def test_rejections():
    k, v, q = _inputs(1, 4, 1, 600, torch.bfloat16, seed=7)
    idx = mp.build_index(k, 13, 20, 3)
    assert mp.capi.mp_tables_workspace_bytes(idx.handle) == 0
    with pytest.raises(ValueError):
        mp.build_tables(idx)
    small = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(mp.MPError, match="MP_E_SHAPE"):
        mp.capi.mp_build_tables(idx.handle, small.data_ptr(), small.numel(), 0)
    idx2 = mp.build_index(k, 8, 20, 3)
    with pytest.raises(mp.MPError, match="MP_E_ARG"):
        mp.decode_attn_tables(q, idx2, k, v, 4, 16, scratch=torch.empty(
            idx2.scratch_bytes(4, tables=True), dtype=torch.uint8, device=DEV))
    with pytest.raises(mp.MPError, match="MP_E_WORKSPACE"):
        mp.capi.mp_build_tables(idx2.handle, small.data_ptr(), small.numel(), 0)


def test_largest_n_the_tables_take_at_L255():
    """The collision bitmap of a head (2 bits per key) must fit in a
    workgroup's LDS beside 2L + 1 bucket words: at L = 255 that allows
    n_pad / 4 + 2044 <= 162,816 bytes, i.e. 1256 chunks (643,072 keys).  The
    largest such n decodes exactly like the code scan; one key more is
    refused."""
    n = 1256 * 512
    k, v, q = _inputs(1, 4, 1, n, torch.bfloat16, seed=71)
    r = run_tables_case(k, v, q, 10, 255, seed=71, n_sink=4, n_local=64,
                        heads=[(0, 0), (0, 3)], table_rows=[0, 254])
    print("n = 643,072 at L = 255:", r, flush=True)
    del k, v, q
    k, v, q = _inputs(1, 4, 1, n + 1, torch.bfloat16, seed=72)
    idx = mp.build_index(k, 10, 255, 72)
    assert mp.capi.mp_tables_workspace_bytes(idx.handle) == 0
    with pytest.raises(ValueError):
        mp.build_tables(idx)
