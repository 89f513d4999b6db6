"""Stage-by-stage comparison of the HIP path with the fp64 oracle.

Bars (the method's own statement of parity):
  * hyperplanes: identical fp32 values up to one ulp (host and device libm);
  * mu: within one fp32 ulp of the fp64 mean;
  * key and query codes: bit-exact except bits whose projection lies inside
    |w.x| < 1e-5 |w||x| (the band), and fewer than 0.01% of bits;
  * collision counts and sampled sets: exact, computed by the oracle on the
    GPU's own codes (integer steps);
  * outputs: per (sequence, head) row, max|o_gpu - o_ref| / max|o_ref| <= 2e-3.

Every key of every (sequence, KV head) and every query head is checked.
Beside the bars, run_case reports what the band allows to differ: the keys
whose membership in S changes when the oracle runs its integer steps on its
own codes instead of the GPU's (each must trace back to a code bit that
differs, and every differing bit lies in the band), and the output error
against the oracle's estimate on its own S.  With MP_PARITY_REPORT set to a
file path, each report is appended there as one JSON line.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import lsh_sampled_sparse_amd as mp
import oracle

OUT_TOL = 2e-3
BAND_CAP = 1e-4


def oracle_threads() -> int:
    """Threads for the oracle's key encode: the CPU share of the process."""
    env = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return env if env > 0 else min(16, os.cpu_count() or 1)


def ulp_distance_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = a.astype(np.float32).view(np.int32).astype(np.int64)
    bi = b.astype(np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, np.int64(-2**31) - ai, ai)
    bi = np.where(bi < 0, np.int64(-2**31) - bi, bi)
    return np.abs(ai - bi)


def unpack_planes(planes: np.ndarray, K: int, L: int, n: int) -> np.ndarray:
    """Codes [L][n] uint16 of one (sequence, KV head) from its bit planes
    [nc][L*max(K,1)][16] uint32: bit j of word w of row l*K + b is bit b of
    the table-l code of key 32w + j of the chunk."""
    nc, rows, words = planes.shape
    Kr = max(K, 1)
    assert rows == L * Kr and words * 32 == mp.MP_CHUNK
    by = np.ascontiguousarray(planes.astype("<u4")).view(np.uint8).reshape(nc, L, Kr, words * 4)
    bits = np.unpackbits(by, axis=-1, bitorder="little")          # [nc][L][Kr][512]
    codes = np.zeros((nc, L, mp.MP_CHUNK), dtype=np.uint16)
    for b in range(K):
        codes |= bits[:, :, b, :].astype(np.uint16) << b
    return codes.transpose(1, 0, 2).reshape(L, nc * mp.MP_CHUNK)[:, :n]


def gpu_codes_table_major(idx: mp.MagicPIGIndex) -> np.ndarray:
    """[B][H_kv][L][n] uint16 from the device's bit planes."""
    _, _, planes = idx.views()
    p = planes.cpu().numpy().view(np.uint32)            # [B][H][nc][L*Kr][16]
    B, H = p.shape[:2]
    out = np.empty((B, H, idx.L, idx.n), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            out[b, h] = unpack_planes(p[b, h], idx.K, idx.L, idx.n)
    return out


def check_codes(ref_vecs: np.ndarray, W: np.ndarray, K: int, L: int, got: np.ndarray, what: str):
    """One vector at a time: ref_vecs [m][d] fp64 (already centered for
    keys); got [m][L] uint16.  Returns (mismatched bits, band bits, total
    bits); raises on a mismatch outside the band or above the cap."""
    m = ref_vecs.shape[0]
    mism = band_total = 0
    for i in range(m):
        code, band = oracle.encode(ref_vecs[i], W, K, L)
        band_total += int(band.sum())
        x = code ^ got[i]
        if not x.any():
            continue
        for l in np.nonzero(x)[0]:
            for b in range(K):
                if (int(x[l]) >> b) & 1:
                    mism += 1
                    assert band[l * K + b], f"{what} {i} table {l} bit {b} differs outside the band"
    bits = m * K * L
    if bits:
        assert mism <= BAND_CAP * bits + 1e-9 or mism <= 1, f"{what}: {mism} of {bits} bits differ"
    return mism, band_total, bits


def check_unit_codes(ref: np.ndarray, band: np.ndarray, got: np.ndarray, what: str):
    """Whole-unit code check, ref/band/got [L][n] uint16 (band: the mask of
    bits inside the band).  Returns (mismatched bits, band bits)."""
    x = ref ^ got
    outside = x & ~band
    if outside.any():
        l, i = np.argwhere(outside)[0]
        raise AssertionError(f"{what}: key {i} table {l} differs outside the band "
                             f"(gpu {got[l, i]:#x}, oracle {ref[l, i]:#x}, band {band[l, i]:#x})")
    return int(np.bitwise_count(x).sum()), int(np.bitwise_count(band).sum())


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.max(np.abs(ref))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def elem_rel_err(got: np.ndarray, ref: np.ndarray, floor: float = 1e-3) -> float:
    """Largest elementwise error relative to max(|ref_j|, floor * max|ref|):
    a reported companion to row_rel_err (the bar), which near-zero elements
    would make unstable without the floor."""
    top = np.max(np.abs(ref))
    if top == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor * top)))


def write_report(name: str, rep: dict):
    path = os.environ.get("MP_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": name, **rep}) + "\n")


def run_case(k, v, q, K, L, seed, n_sink, n_local, scale=0.0, name=None, idx=None):
    """Run build + decode_debug on the GPU and check every stage of every
    (sequence, KV head) unit and every query head against the oracle.
    `idx`: an index already built from k (default: built here)."""
    B, H_kv, n, d = k.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    own_idx = idx is None
    if own_idx:
        idx = mp.build_index(k, K, L, seed)
    res = mp.decode_debug(q, idx, k, v, n_sink, n_local, scale=scale)
    out2 = mp.decode_attn(q, idx, k, v, n_sink, n_local, scale=scale)
    torch.cuda.synchronize()
    # production path and debug path agree bit for bit
    assert torch.equal(res["out"], out2), "mp_decode_attn and mp_decode_debug outputs differ"

    W_gpu, mu_gpu, _ = idx.views()
    W_gpu = W_gpu.cpu().numpy()
    W = oracle.hyperplanes(seed, K * L, d)
    du = ulp_distance_f32(W, W_gpu)
    rep = {"W_diff": int(np.count_nonzero(du))}
    assert du.max(initial=0) <= 1 and rep["W_diff"] <= max(1, 1e-5 * W.size)
    codes = gpu_codes_table_major(idx)
    qcodes = res["qcodes"].cpu().numpy().view(np.uint16)
    counts = res["counts"].cpu().numpy()
    s_idx = res["s_idx"].cpu().numpy()
    s_len = res["s_len"].cpu().numpy()
    out = res["out"].cpu().double().numpy()
    mu_gpu = mu_gpu.cpu().numpy()
    scl = scale if scale > 0 else 1.0 / math.sqrt(d)
    key_mism = key_band = q_mism = q_band = 0
    s_diff_keys = s_diff_heads = 0
    errs, errs_own, errs_elem = [], [], []
    threads = oracle_threads()
    for b in range(B):
        for h in range(H_kv):
            kh = k[b, h].cpu().double().numpy()
            vh = v[b, h].cpu().double().numpy()
            mu = oracle.mean(kh)
            assert ulp_distance_f32(mu.astype(np.float32), mu_gpu[b, h]).max() <= 1
            ref_codes, band, _ = oracle.encode_keys_band_parallel(kh, W, K, L, mu, threads)
            m_, b_ = check_unit_codes(ref_codes, band, codes[b, h], f"key codes ({b},{h})")
            key_mism += m_
            key_band += b_
            for g in range(G):
                hq = h * G + g
                qh = q[b, hq].cpu().double().numpy()
                qref, qband = oracle.encode(qh, W, K, L)
                m_, _, _ = check_codes(qh[None], W, K, L, qcodes[b, hq][None], "query")
                q_mism += m_
                q_band += int(qband.sum())
                # integer steps on the GPU's codes: exact
                cnt = oracle.collision_counts(codes[b, h], qcodes[b, hq])
                assert np.array_equal(cnt, counts[b, hq].astype(np.int32)), \
                    f"counts differ at (b={b}, h={hq})"
                S = oracle.select(cnt, n_sink, n_local)
                assert s_len[b, hq] == len(S), f"|S| differs at (b={b}, h={hq})"
                assert np.array_equal(S, s_idx[b, hq, :len(S)]), f"S differs at (b={b}, h={hq})"
                ref = oracle.estimate(qh, kh, vh, mu, S, K, L, n_sink, n_local, scl)
                e = row_rel_err(out[b, hq], ref)
                errs.append(e)
                errs_elem.append(elem_rel_err(out[b, hq], ref))
                assert e <= OUT_TOL, f"output error {e:.3g} at (b={b}, h={hq})"
                # the oracle's integer steps on its own codes: S may differ
                # only at keys where a code bit differs (in the band)
                S_own = oracle.select(oracle.collision_counts(ref_codes, qref), n_sink, n_local)
                diff = np.setxor1d(S, S_own)
                if diff.size:
                    s_diff_heads += 1
                    s_diff_keys += int(diff.size)
                    qdiff = bool((qref != qcodes[b, hq]).any())
                    for i in diff:
                        assert qdiff or (ref_codes[:, i] != codes[b, h][:, i]).any(), \
                            f"key {i} of head ({b},{hq}) changes S with no differing code"
                    ref_own = oracle.estimate(qh, kh, vh, mu, S_own, K, L, n_sink, n_local, scl)
                    errs_own.append(row_rel_err(out[b, hq], ref_own))
                else:
                    errs_own.append(e)
    key_bits = B * H_kv * n * K * L
    q_bits = B * H_q * K * L
    assert key_mism <= BAND_CAP * key_bits or key_mism <= 1, \
        f"{key_mism} of {key_bits} key bits differ"
    rep.update(keys_checked=B * H_kv * n, key_bits=key_bits, key_mismatched_bits=key_mism,
               key_band_bits=key_band, heads_checked=B * H_q, query_bits=q_bits,
               query_mismatched_bits=q_mism, query_band_bits=q_band,
               max_out_err=max(errs) if errs else 0.0,
               max_out_err_elementwise=max(errs_elem) if errs_elem else 0.0,
               s_diff_vs_oracle_codes={"heads": s_diff_heads, "keys": s_diff_keys},
               max_out_err_vs_oracle_own_S=max(errs_own) if errs_own else 0.0,
               mean_S=float(s_len.mean()))
    # legacy keys read by callers
    rep["mismatched_bits"] = key_mism + q_mism
    rep["bits"] = key_bits + q_bits
    if name:
        write_report(name, rep)
    if own_idx:
        del idx
    return rep
