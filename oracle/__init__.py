"""fp64 CPU oracle of MagicPIG's decode-time attention estimator (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of bench.py import this.  The HIP path never does, and this
package imports nothing from it.

Every function takes and returns numpy arrays; floating inputs are converted
to float64 exactly (bf16 and fp32 values are exact in fp64).  The arithmetic
lives in oracle.c, which cites the pages each step follows:
  * "MagicPIG: don't pick the tallest", sections 5-6;
  * "MagicPIG: LSH Sampling for Efficient LLM Generation", background
    (SimHash), method details (estimator, u_i, centering, algorithm steps)
    and system co-design (exact sink/local tokens).
"""

from __future__ import annotations

import ctypes as C
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MP_ORACLE_LIB names another build of oracle.c (the sanitized one of
# build.build(sanitize=True)); the default is the plain build beside this file.
_LIB_PATH = os.environ.get("MP_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

SCORE_CENTERED = 1
CONST_LOG_U = 2
AUGMENTED = 4

_dp = C.POINTER(C.c_double)
_fp = C.POINTER(C.c_float)
_u8p = C.POINTER(C.c_uint8)
_u16p = C.POINTER(C.c_uint16)
_i32p = C.POINTER(C.c_int32)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.orc_splitmix64.restype = C.c_uint64
        L.orc_splitmix64.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_gauss.restype = C.c_double
        L.orc_gauss.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_hyperplanes.restype = None
        L.orc_hyperplanes.argtypes = [C.c_uint64, C.c_int64, C.c_int64, C.c_int, _fp]
        L.orc_mean.restype = None
        L.orc_mean.argtypes = [_dp, C.c_int64, C.c_int, _dp]
        L.orc_project_signs.restype = None
        L.orc_project_signs.argtypes = [_dp, C.c_int, _fp, C.c_int64, _u8p, _u8p]
        L.orc_pack_codes.restype = None
        L.orc_pack_codes.argtypes = [_u8p, C.c_int, C.c_int, _u16p]
        L.orc_encode.restype = C.c_int64
        L.orc_encode.argtypes = [_dp, C.c_int, _fp, C.c_int, C.c_int, _u16p, _u8p]
        L.orc_encode_keys.restype = C.c_int64
        L.orc_encode_keys.argtypes = [_dp, C.c_int64, C.c_int, _dp, _fp, C.c_int, C.c_int, _u16p]
        L.orc_encode_keys_band.restype = C.c_int64
        L.orc_encode_keys_band.argtypes = [_dp, C.c_int64, C.c_int, _dp, _fp, C.c_int, C.c_int,
                                           _u16p, _u16p]
        L.orc_collision_counts.restype = None
        L.orc_collision_counts.argtypes = [_u16p, C.c_int64, C.c_int, _u16p, _i32p]
        L.orc_select.restype = C.c_int64
        L.orc_select.argtypes = [_i32p, C.c_int64, C.c_int64, C.c_int64, _i32p]
        L.orc_log_u.restype = C.c_double
        L.orc_log_u.argtypes = [C.c_double, C.c_int, C.c_int]
        L.orc_u.restype = C.c_double
        L.orc_u.argtypes = [C.c_double, C.c_int, C.c_int]
        L.orc_collision_p.restype = C.c_double
        L.orc_collision_p.argtypes = [_dp, _dp, C.c_int]
        L.orc_estimate.restype = C.c_int
        L.orc_estimate.argtypes = [_dp, _dp, _dp, _dp, C.c_int64, C.c_int, C.c_int, C.c_int,
                                   _i32p, C.c_int64, C.c_int64, C.c_int64, C.c_double, C.c_int,
                                   C.c_double, C.c_double, _dp]
        L.orc_aug_radius.restype = C.c_double
        L.orc_aug_radius.argtypes = [_dp, C.c_int64, C.c_int, _dp]
        L.orc_hyperplane_extra.restype = None
        L.orc_hyperplane_extra.argtypes = [C.c_uint64, C.c_int64, C.c_int, _fp]
        L.orc_encode_keys_aug.restype = C.c_int64
        L.orc_encode_keys_aug.argtypes = [_dp, C.c_int64, C.c_int, _dp, _fp, _fp, C.c_double,
                                          C.c_int, C.c_int, _u16p]
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _f64(a):
    if hasattr(a, "detach"):          # torch tensor
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------- hyperplanes
def splitmix64(seed: int, k: int) -> int:
    return int(lib().orc_splitmix64(seed & (2**64 - 1), k))


def gauss(seed: int, e: int) -> float:
    return float(lib().orc_gauss(seed & (2**64 - 1), e))


def hyperplanes(seed: int, R: int, d: int, row0: int = 0) -> np.ndarray:
    W = np.empty((R, d), dtype=np.float32)
    if R:
        lib().orc_hyperplanes(seed & (2**64 - 1), row0, R, d, _p(W, _fp))
    return W


# ----------------------------------------------------------------- centering
def mean(keys) -> np.ndarray:
    k = _f64(keys)
    n, d = k.shape
    mu = np.empty(d, dtype=np.float64)
    lib().orc_mean(_p(k, _dp), n, d, _p(mu, _dp))
    return mu


# ------------------------------------------------------------------- SimHash
def project_signs(x, W):
    x = _f64(x)
    W = np.ascontiguousarray(W, dtype=np.float32)
    R, d = W.shape
    bits = np.empty(R, dtype=np.uint8)
    band = np.empty(R, dtype=np.uint8)
    lib().orc_project_signs(_p(x, _dp), d, _p(W, _fp), R, _p(bits, _u8p), _p(band, _u8p))
    return bits, band


def pack_codes(bits, K, L):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    code = np.empty(L, dtype=np.uint16)
    lib().orc_pack_codes(_p(bits, _u8p), K, L, _p(code, _u16p))
    return code


def encode(x, W, K, L):
    """Codes [L] and band flags [K*L] of one (already centered, or raw) vector."""
    x = _f64(x)
    W = np.ascontiguousarray(W, dtype=np.float32)
    code = np.empty(max(L, 1), dtype=np.uint16)
    band = np.empty(max(K * L, 1), dtype=np.uint8)
    lib().orc_encode(_p(x, _dp), x.shape[0], _p(W, _fp), K, L, _p(code, _u16p), _p(band, _u8p))
    return code[:L], band[:K * L]


def encode_keys(keys, W, K, L, mu=None):
    """Table-major codes [L][n] of k_i - mu (raw keys if mu is None); band count."""
    k = _f64(keys)
    n, d = k.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    codes = np.empty((L, n), dtype=np.uint16)
    mup = None
    if mu is not None:
        mu = _f64(mu)
        mup = _p(mu, _dp)
    nb = lib().orc_encode_keys(_p(k, _dp), n, d, mup, _p(W, _fp), K, L, _p(codes, _u16p))
    return codes, int(nb)


def encode_keys_parallel(keys, W, K, L, mu=None, threads=None):
    """Same as encode_keys, split over row blocks in threads (ctypes drops the GIL)."""
    k = _f64(keys)
    n = k.shape[0]
    threads = threads or os.cpu_count() or 1
    if threads <= 1 or n < 256:
        return encode_keys(k, W, K, L, mu)
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda t: encode_keys(k[bounds[t]:bounds[t + 1]], W, K, L, mu),
                            range(threads)))
    codes = np.concatenate([p[0] for p in parts], axis=1)
    return codes, sum(p[1] for p in parts)


def encode_keys_band(keys, W, K, L, mu=None):
    """Table-major codes [L][n] of k_i - mu and the band masks [L][n] (bit b of
    band[l][i] set where hyperplane l*K + b projects key i inside the 1e-5
    band); band count."""
    k = _f64(keys)
    n, d = k.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    codes = np.empty((L, n), dtype=np.uint16)
    band = np.empty((L, n), dtype=np.uint16)
    mup = None
    if mu is not None:
        mu = _f64(mu)
        mup = _p(mu, _dp)
    nb = lib().orc_encode_keys_band(_p(k, _dp), n, d, mup, _p(W, _fp), K, L, _p(codes, _u16p),
                                    _p(band, _u16p))
    return codes, band, int(nb)


def encode_keys_band_parallel(keys, W, K, L, mu=None, threads=None):
    """encode_keys_band split over row blocks in threads (ctypes drops the GIL)."""
    k = _f64(keys)
    n = k.shape[0]
    threads = threads or os.cpu_count() or 1
    if threads <= 1 or n < 256:
        return encode_keys_band(k, W, K, L, mu)
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda t: encode_keys_band(k[bounds[t]:bounds[t + 1]], W, K, L, mu),
                            range(threads)))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1), sum(p[2] for p in parts))


# ----------------------------------------------------------- sampling rule
def collision_counts(codes, qcode):
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    qcode = np.ascontiguousarray(qcode, dtype=np.uint16)
    L, n = codes.shape
    counts = np.empty(n, dtype=np.int32)
    lib().orc_collision_counts(_p(codes, _u16p), n, L, _p(qcode, _u16p), _p(counts, _i32p))
    return counts


def select(counts, n_sink, n_local):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    n = counts.shape[0]
    idx = np.empty(max(n, 1), dtype=np.int32)
    m = lib().orc_select(_p(counts, _i32p), n, n_sink, n_local, _p(idx, _i32p))
    return idx[:m].copy()


# ------------------------------------------------------ collision probability
def log_u(p: float, K: int, L: int) -> float:
    return float(lib().orc_log_u(float(p), K, L))


def u(p: float, K: int, L: int) -> float:
    return float(lib().orc_u(float(p), K, L))


def collision_p(a, b) -> float:
    a = _f64(a)
    b = _f64(b)
    return float(lib().orc_collision_p(_p(a, _dp), _p(b, _dp), a.shape[0]))


# --------------------------------------------------------------- estimator
def estimate(q, keys, values, mu, S, K, L, n_sink, n_local, scale=None, flags=0,
             const_log_u=0.0, aug_r=None):
    """flags: SCORE_CENTERED, CONST_LOG_U; aug_r (the augmentation radius)
    switches p_i to the lifted pair, see aug_radius."""
    q = _f64(q)
    k = _f64(keys)
    v = _f64(values)
    n, d = k.shape
    S = np.ascontiguousarray(S, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty(d, dtype=np.float64)
    mup = None
    if mu is not None:
        mu = _f64(mu)
        mup = _p(mu, _dp)
    Sp = _p(S, _i32p) if S.size else None
    rc = lib().orc_estimate(_p(q, _dp), _p(k, _dp), _p(v, _dp), mup, n, d, K, L, Sp, S.size,
                            n_sink, n_local, float(scale),
                            flags | (AUGMENTED if aug_r is not None else 0), float(const_log_u),
                            float(aug_r or 0.0), _p(out, _dp))
    if rc != 0:
        raise ValueError(f"orc_estimate failed with status {rc}")
    return out


# ------------------------------------------------ inner-product-to-cosine augmentation
def aug_radius(keys, mu=None) -> float:
    """r = max_i |k_i - mu| (the norm every lifted key gets)."""
    k = _f64(keys)
    mup = None if mu is None else _p(_f64(mu), _dp)
    return float(lib().orc_aug_radius(_p(k, _dp), k.shape[0], k.shape[1], mup))


def hyperplane_extra(seed: int, R: int, d: int) -> np.ndarray:
    """The lifted coordinate w_j of hyperplanes j < R (normal numbers R*d + j)."""
    w = np.empty(R, dtype=np.float32)
    lib().orc_hyperplane_extra(seed, R, d, _p(w, _fp))
    return w


def encode_keys_aug(keys, W, w, K, L, mu, r):
    """Table-major codes [L][n] of the lifted keys [k - mu, sqrt(r^2 - |k - mu|^2)]
    against the lifted hyperplanes [W_j, w_j]; band count."""
    k = _f64(keys)
    n, d = k.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    codes = np.empty((L, n), dtype=np.uint16)
    mup = None if mu is None else _p(_f64(mu), _dp)
    nb = lib().orc_encode_keys_aug(_p(k, _dp), n, d, mup, _p(W, _fp), _p(w, _fp), float(r), K, L,
                                   _p(codes, _u16p))
    return codes, int(nb)


# ------------------------------------------------ whole-unit convenience
def decode_unit(q_heads, keys, values, W, K, L, n_sink, n_local, scale=None, centered=True,
                codes=None, mu=None):
    """All steps for one KV head and its G query heads.

    q_heads [G][d]; keys/values [n][d].  Returns dict with mu, codes [L][n],
    band, qcodes [G][L], counts [G][n], S (list of arrays), out [G][d].
    ``codes``/``mu`` may be passed in to skip the key encode.
    """
    k = _f64(keys)
    if mu is None:
        mu = mean(k) if centered else None
    band = None
    if codes is None:
        codes, band = encode_keys_parallel(k, W, K, L, mu if centered else None)
    qh = _f64(q_heads)
    G = qh.shape[0]
    qcodes = np.empty((G, L), dtype=np.uint16)
    counts = np.empty((G, k.shape[0]), dtype=np.int32)
    S, outs = [], np.empty((G, k.shape[1]), dtype=np.float64)
    for g in range(G):
        qcodes[g], _ = encode(qh[g], W, K, L)
        counts[g] = collision_counts(codes, qcodes[g])
        S.append(select(counts[g], n_sink, n_local))
        outs[g] = estimate(qh[g], k, values, mu if centered else None, S[-1], K, L,
                           n_sink, n_local, scale)
    return dict(mu=mu, codes=codes, band=band, qcodes=qcodes, counts=counts, S=S, out=outs)
