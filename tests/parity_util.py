"""Stage-by-stage comparison of the HIP path with the fp64 oracle.

Bars (the method's own statement of parity):
  * hyperplanes: identical fp32 values up to one ulp (host and device libm);
  * mu: within one fp32 ulp of the fp64 mean;
  * key and query codes: bit-exact except bits whose projection lies inside
    |w.x| < 1e-5 |w||x| (the band), and fewer than 0.01% of bits;
  * collision counts and sampled sets: exact, computed by the oracle on the
    GPU's own codes (integer steps);
  * outputs: per (sequence, head) row, max|o_gpu - o_ref| / max|o_ref| <= 2e-3.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import lsh_sampled_sparse_amd as mp
import oracle

OUT_TOL = 2e-3
BAND_CAP = 1e-4


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
    """ref_vecs [m][d] fp64 (already centered for keys); got [m][L] uint16.
    Returns (mismatched bits, band bits, total bits); raises on a mismatch
    outside the band or above the cap."""
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


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.max(np.abs(ref))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def run_case(k, v, q, K, L, seed, n_sink, n_local, scale=0.0, heads=None, key_rows=None,
             check_all_codes=True):
    """Run build + decode_debug on the GPU and check every stage against the
    oracle.  heads: optional list of (b, hq) to check outputs for (all by
    default); key_rows: optional key subset for the code comparison."""
    B, H_kv, n, d = k.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    idx = mp.build_index(k, K, L, seed)
    res = mp.decode_debug(q, idx, k, v, n_sink, n_local, scale=scale)
    out2 = mp.decode_attn(q, idx, k, v, n_sink, n_local, scale=scale)
    torch.cuda.synchronize()
    report = {}
    # production path and debug path agree bit for bit
    assert torch.equal(res["out"], out2), "mp_decode_attn and mp_decode_debug outputs differ"

    W_gpu, mu_gpu, _ = idx.views()
    W_gpu = W_gpu.cpu().numpy()
    W = oracle.hyperplanes(seed, K * L, d)
    du = ulp_distance_f32(W, W_gpu)
    report["W_diff"] = int(np.count_nonzero(du))
    assert du.max(initial=0) <= 1 and report["W_diff"] <= max(1, 1e-5 * W.size)
    codes = gpu_codes_table_major(idx)
    qcodes = res["qcodes"].cpu().numpy().view(np.uint16)
    counts = res["counts"].cpu().numpy().astype(np.int32)
    s_idx = res["s_idx"].cpu().numpy()
    s_len = res["s_len"].cpu().numpy()
    out = res["out"].cpu().double().numpy()
    mu_gpu = mu_gpu.cpu().numpy()
    scl = scale if scale > 0 else 1.0 / math.sqrt(d)
    mism = bits = 0
    errs = []
    for b in range(B):
        for h in range(H_kv):
            kh = k[b, h].cpu().double().numpy()
            vh = v[b, h].cpu().double().numpy()
            mu = oracle.mean(kh)
            assert ulp_distance_f32(mu.astype(np.float32), mu_gpu[b, h]).max() <= 1
            rows = np.arange(n) if key_rows is None else key_rows
            if check_all_codes or key_rows is not None:
                m_, _, b_ = check_codes(kh[rows] - mu, W, K, L, codes[b, h][:, rows].T, "key")
                mism += m_
                bits += b_
            for g in range(G):
                hq = h * G + g
                if heads is not None and (b, hq) not in heads:
                    continue
                qh = q[b, hq].cpu().double().numpy()
                m_, _, b_ = check_codes(qh[None], W, K, L, qcodes[b, hq][None], "query")
                mism += m_
                bits += b_
                cnt = oracle.collision_counts(codes[b, h], qcodes[b, hq])
                assert np.array_equal(cnt, counts[b, hq]), f"counts differ at (b={b}, h={hq})"
                S = oracle.select(cnt, n_sink, n_local)
                assert s_len[b, hq] == len(S), f"|S| differs at (b={b}, h={hq})"
                assert np.array_equal(S, s_idx[b, hq, :len(S)]), f"S differs at (b={b}, h={hq})"
                ref = oracle.estimate(qh, kh, vh, mu, S, K, L, n_sink, n_local, scl)
                e = row_rel_err(out[b, hq], ref)
                errs.append(e)
                assert e <= OUT_TOL, f"output error {e:.3g} at (b={b}, h={hq})"
    report.update(mismatched_bits=mism, bits=bits, max_out_err=max(errs) if errs else 0.0,
                  mean_S=float(s_len.mean()))
    del idx
    return report
