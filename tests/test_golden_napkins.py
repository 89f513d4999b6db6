"""The byte and entry figures that the page "MagicPIG: don't pick the tallest"
prints (section 1: KV bytes per token of Llama-3.1-8B at a 96K context;
section 6 "The bill": table entries per token and per query at K=10, L=150),
stored in tests/golden/page_napkins.json, against:
  * their own arithmetic (the stored numbers follow from the model shape);
  * the 96K workload the benchmark times (same model shape and (K, L));
  * the index size the library reports (K-bit codes per table, the page's
    packed hash bits, instead of its 32-bit token index per table entry);
  * the oracle's encoder and collision counts: a query's bucket in one table
    holds sum_i p_i^K keys in expectation over the hyperplanes, with
    p_i = 1 - theta_i/pi (page "MagicPIG: LSH Sampling for Efficient LLM
    Generation", background: SimHash agreement probability).  The page's
    L n / 2^K figure is that expectation for evenly filled buckets.
CPU only."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from lsh_sampled_sparse_amd import capi

GOLD = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                   "page_napkins.json")))


def test_page_figures_follow_from_the_model_shape():
    m = GOLD["llama31_8b"]
    per_token = m["layers"] * m["kv_heads"] * m["head_dim"] * 2 * m["bytes_per_elem"]
    assert per_token == GOLD["kv_bytes_per_token"]
    assert per_token * m["context"] / 2**30 == pytest.approx(GOLD["kv_bytes_total_gib"], abs=0.05)
    # a 32-bit token index per table and token
    assert GOLD["L"] * 4 == GOLD["table_bytes_per_token_per_head_layer"]
    tables = GOLD["table_bytes_per_token_per_head_layer"] * m["context"] * m["layers"] * \
        m["kv_heads"]
    assert tables / 2**30 == pytest.approx(GOLD["tables_total_gib"], abs=0.05)
    entries = GOLD["L"] * m["context"] / 2**GOLD["K"]
    assert entries == GOLD["entries_scanned_per_query"]
    assert entries * 4 == GOLD["index_bytes_scanned_per_query"]
    key_bytes = m["context"] * m["head_dim"] * m["bytes_per_elem"]
    assert key_bytes == GOLD["key_bytes_one_head_one_layer"]
    assert 100 * entries * 4 / key_bytes == pytest.approx(GOLD["scanned_fraction_percent"],
                                                          abs=0.005)


def test_timed_workload_is_the_pages_model():
    m = GOLD["llama31_8b"]
    cfg = synth.CONFIGS["llama8b_96k"]
    assert (cfg.n, cfg.H_kv, cfg.d, cfg.layers) == (m["context"], m["kv_heads"], m["head_dim"],
                                                   m["layers"])
    assert torch.empty(0, dtype=cfg.dtype).element_size() == m["bytes_per_elem"]
    assert (cfg.K, cfg.L) == (GOLD["K"], GOLD["L"])
    assert cfg.H_kv * cfg.n * cfg.d * 2 * m["bytes_per_elem"] * cfg.layers == \
        GOLD["kv_bytes_per_token"] * cfg.n


def test_index_bytes_against_the_pages_tables():
    m = GOLD["llama31_8b"]
    n, H, K, L = m["context"], m["kv_heads"], GOLD["K"], GOLD["L"]
    total = capi.mp_index_workspace_bytes(1, H, n, 128, K, L)
    codes = H * n * L * K // 8                  # K bits per table, key and KV head
    # a 32-bit table entry per table and token is 32/K times the packed code
    assert codes * 32 == H * n * GOLD["table_bytes_per_token_per_head_layer"] * K
    # the rest is W (two copies, fp32), mu and the fp64 partial sums of the mean
    assert 0 <= total - codes < 4 << 20


@pytest.mark.parametrize("seed", [1000, 1001])
def test_bucket_occupancy_matches_simhash_expectation(seed):
    K, L, n, G = GOLD["K"], GOLD["L"], 16384, 4
    inp = synth.cone_inputs(B=1, H_q=G, H_kv=1, n=n, d=128, dtype=torch.bfloat16, seeds=[seed])
    keys = inp["k"][0, 0].double().numpy()
    qs = inp["q"][0].double().numpy()
    W = oracle.hyperplanes(seed, K * L, 128)
    mu = oracle.mean(keys)
    codes, _ = oracle.encode_keys_parallel(keys, W, K, L, mu, threads=8)
    x = keys - mu
    xn = np.linalg.norm(x, axis=1)
    for g in range(G):
        qc, _ = oracle.encode(qs[g], W, K, L)
        bucket = (codes == qc[:, None]).sum(axis=1)          # keys in q's bucket, per table
        assert bucket.sum() == oracle.collision_counts(codes, qc).sum()
        cos = np.clip(x @ qs[g] / (xn * np.linalg.norm(qs[g])), -1.0, 1.0)
        expect = np.sum((1.0 - np.arccos(cos) / math.pi) ** K)
        se = bucket.std(ddof=1) / math.sqrt(L)            # tables are independent draws
        print(f"seed {seed} head {g}: mean bucket {bucket.mean():.1f}, "
              f"sum p^K {expect:.1f}, even buckets n/2^K {n / 2**K:.1f}")
        assert abs(bucket.mean() - expect) < 5 * se
