"""Pins of the fp64 oracle against facts other than itself (CPU only).

Each test ties one oracle step to something the pages or mathematics fix:
  * SimHash agreement 1 - theta/pi (page "MagicPIG: LSH Sampling for
    Efficient LLM Generation", background section; page "MagicPIG: don't pick
    the tallest", section 5) -- Monte Carlo;
  * u_i, the chance of colliding in at least 2 of L tables (same pages,
    method details / section 5) -- brute-force enumeration over tables, exact
    rational binomial tails, closed-form corners, Monte Carlo over seeds;
  * the estimator reduces to exact softmax attention when every key is sampled
    with one constant u -- torch float64 softmax;
  * convergence to exact attention as L grows;
  * set-inclusion semantics (page "MagicPIG: don't pick the tallest", sec. 5):
    Horvitz-Thompson unbiasedness of both sums of the ratio;
  * centering leaves the output unchanged, and without it the sampled set
    collapses (same page, section 5; method details of the summary page);
  * the fraction of projections inside the 1e-5 band against its closed form;
  * integer steps against numpy brute force.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

THETAS = [0.0, math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3, 5 * math.pi / 6,
          math.pi - 0.01]


# ---------------------------------------------------------------- RNG
def test_splitmix64_reference_stream():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "splitmix64_seed1234567.json")))
    got = [oracle.splitmix64(g["seed"], k) for k in range(1, 6)]
    assert got == g["outputs"]


def test_hyperplanes_standard_normal_and_row_indexed():
    from scipy import stats
    W = oracle.hyperplanes(seed=5, R=8192, d=128).astype(np.float64).ravel()
    N = W.size
    assert abs(W.mean()) < 5.0 / math.sqrt(N)
    assert abs(W.var() - 1.0) < 5.0 * math.sqrt(2.0 / N)
    assert abs(stats.kurtosis(W, fisher=False) - 3.0) < 5.0 * math.sqrt(24.0 / N)
    assert stats.kstest(W, "norm").pvalue > 1e-4
    # a row block generated on its own equals the same rows of a longer matrix
    full = oracle.hyperplanes(seed=9, R=40, d=16)
    part = oracle.hyperplanes(seed=9, R=10, d=16, row0=25)
    assert np.array_equal(full[25:35], part)
    # different seeds give different streams
    assert not np.array_equal(full, oracle.hyperplanes(seed=10, R=40, d=16))


# ---------------------------------------------------------------- SimHash
@pytest.mark.parametrize("d,R", [(2, 10**6), (16, 10**6), (128, 4 * 10**5)])
def test_simhash_agreement_is_one_minus_theta_over_pi(d, R):
    rng = np.random.default_rng(100 + d)
    Q, _ = np.linalg.qr(rng.standard_normal((d, 2)))
    e1, e2 = Q[:, 0], Q[:, 1]
    ys = [math.cos(t) * e1 + math.sin(t) * e2 for t in THETAS]
    agree = np.zeros(len(THETAS))
    chunk = 100_000
    for r0 in range(0, R, chunk):
        W = oracle.hyperplanes(seed=777 + d, R=min(chunk, R - r0), d=d, row0=r0)
        bx, _ = oracle.project_signs(1.7 * e1, W)
        for t, y in enumerate(ys):
            by, _ = oracle.project_signs(y, W)
            agree[t] += np.count_nonzero(bx == by)
    for t, theta in enumerate(THETAS):
        p = 1.0 - theta / math.pi
        sigma = math.sqrt(max(p * (1 - p), 1e-12) / R)
        assert abs(agree[t] / R - p) <= 5 * sigma + 1e-12, (d, theta, agree[t] / R, p)


def test_project_signs_on_basis_vectors():
    """x = e_c projects onto column c of W: bit j is [W[j][c] > 0]."""
    W = oracle.hyperplanes(seed=3, R=60, d=16)
    for c in (0, 7, 15):
        x = np.zeros(16)
        x[c] = 2.5
        bits, band = oracle.project_signs(x, W)
        assert np.array_equal(bits, (W[:, c] > 0).astype(np.uint8))
        assert not band.any()
    # a zero vector projects to 0 everywhere: sign(0) = 0 (strict inequality)
    bits, _ = oracle.project_signs(np.zeros(16), W)
    assert not bits.any()


def test_pack_codes_lsb_first():
    assert list(oracle.pack_codes([1, 0, 1, 1, 0, 0, 0, 1], 4, 2)) == [13, 8]
    assert list(oracle.pack_codes([], 0, 3)) == [0, 0, 0]       # K = 0: one bucket


# ---------------------------------------------------------------- u_i
def _brute_u(P, L):
    """Sum over all 2^L hit patterns of the L tables with >= 2 hits."""
    pats = np.arange(2 ** L, dtype=np.int64)
    hits = np.zeros_like(pats)
    for b in range(L):
        hits += (pats >> b) & 1
    probs = np.power(P, hits.astype(np.float64)) * np.power(1.0 - P, (L - hits).astype(np.float64))
    return math.fsum(probs[hits >= 2].tolist())


def test_u_matches_enumeration_over_tables():
    seen_small = seen_large = False
    for p in (0.05, 0.2, 0.5, 0.73, 0.9, 0.99):
        for K in (1, 2, 4, 10):
            for L in (2, 3, 5, 8, 16):
                P = p ** K
                ref = _brute_u(P, L)
                got = oracle.u(p, K, L)
                if L * P > 0.05:
                    seen_large = True
                else:
                    seen_small = True
                assert abs(got - ref) <= 1e-13 * ref, (p, K, L, got, ref)
    assert seen_small and seen_large       # both arithmetic branches exercised


@pytest.mark.parametrize("p,K,L", [(Fraction(3, 10), 10, 150), (Fraction(1, 2), 10, 150),
                                   (Fraction(7, 10), 9, 120), (Fraction(9, 10), 9, 240),
                                   (Fraction(1, 10), 4, 16), (Fraction(2, 5), 9, 60),
                                   (Fraction(99, 100), 10, 150)])
def test_u_matches_exact_rational_binomial_tail(p, K, L):
    P = p ** K
    tail = sum(Fraction(math.comb(L, j)) * P ** j * (1 - P) ** (L - j) for j in range(2, L + 1))
    ref = float(tail)
    assert abs(oracle.u(float(p), K, L) - ref) <= 1e-13 * ref
    assert abs(oracle.log_u(float(p), K, L) - math.log(ref)) <= 1e-12 * max(1.0, abs(math.log(ref)))


def test_u_corner_cases():
    for p in (0.1, 0.5, 0.8):
        assert oracle.u(p, 1, 2) == pytest.approx(p * p, rel=1e-15)
        assert oracle.u(p, 3, 2) == pytest.approx(p ** 6, rel=1e-14)
    assert oracle.u(1.0, 10, 150) == 1.0
    assert oracle.u(0.3, 0, 16) == 1.0       # K = 0: every table collides
    assert oracle.u(0.0, 10, 150) == 0.0
    assert oracle.u(0.5, 4, 100_000) == pytest.approx(1.0, abs=1e-12)
    # u grows with p and with L
    ps = np.linspace(0.01, 0.99, 50)
    us = [oracle.u(p, 10, 150) for p in ps]
    assert all(a < b or (a == b == 1.0) for a, b in zip(us, us[1:]))   # saturates at 1.0
    assert oracle.u(0.6, 10, 60) < oracle.u(0.6, 10, 120) < oracle.u(0.6, 10, 240)


def test_u_monte_carlo_over_seeds():
    """A fixed pair at angle pi/3 collides in >= 2 of L tables with frequency u."""
    d, K, L, R = 16, 3, 6, 20000
    rng = np.random.default_rng(7)
    Q, _ = np.linalg.qr(rng.standard_normal((d, 2)))
    x = Q[:, 0]
    y = math.cos(math.pi / 3) * Q[:, 0] + math.sin(math.pi / 3) * Q[:, 1]
    hit = 0
    for s in range(R):
        W = oracle.hyperplanes(seed=50_000 + s, R=K * L, d=d)
        cx, _ = oracle.encode(x, W, K, L)
        cy, _ = oracle.encode(y, W, K, L)
        hit += int(np.count_nonzero(cx == cy) >= 2)
    u = oracle.u(oracle.collision_p(x, y), K, L)
    assert oracle.collision_p(x, y) == pytest.approx(2.0 / 3.0, rel=1e-12)
    assert abs(hit / R - u) <= 5 * math.sqrt(u * (1 - u) / R)


# ---------------------------------------------------------------- estimator
def _tiny_inputs(seed):
    cfg = synth.CONFIGS["tiny"]
    inp = synth.config_inputs(cfg, layer=seed)
    k = inp["k"][0, 0].double().numpy()
    v = inp["v"][0, 0].double().numpy()
    q = inp["q"][0, 0].double().numpy()
    return k, v, q


def _softmax_attention_torch(q, k, v, rows=None):
    kt, vt, qt = torch.from_numpy(k), torch.from_numpy(v), torch.from_numpy(q)
    if rows is not None:
        kt, vt = kt[rows], vt[rows]
    w = torch.softmax(kt @ qt / math.sqrt(k.shape[1]), dim=0)
    return (w @ vt).numpy()


def test_all_sampled_with_constant_u_is_exact_softmax():
    k, v, q = _tiny_inputs(3)
    ref = _softmax_attention_torch(q, k, v)
    # K = 0: every key shares the query's (single) bucket in all L tables, so
    # S = all keys outside T, and u = 1.
    W = oracle.hyperplanes(seed=3, R=0, d=128)
    res = oracle.decode_unit(q[None], k, v, W, K=0, L=16, n_sink=1, n_local=16)
    assert len(res["S"][0]) == 1024 - 17
    assert np.max(np.abs(res["out"][0] - ref)) <= 1e-12 * np.max(np.abs(ref))
    # with no exact set and every key in S, any constant log u cancels in the ratio
    mu = oracle.mean(k)
    S = np.arange(1024, dtype=np.int32)
    out = oracle.estimate(q, k, v, mu, S, 4, 16, 0, 0, flags=oracle.CONST_LOG_U,
                          const_log_u=-3.7)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))
    # ...whereas the real, key-dependent u does not cancel
    out_u = oracle.estimate(q, k, v, mu, S, 4, 16, 0, 0)
    assert np.max(np.abs(out_u - ref)) > 1e-3 * np.max(np.abs(ref))
    # only T (S empty) is exact attention over T; nothing at all gives 0
    T = list(range(1)) + list(range(1024 - 16, 1024))
    out_t = oracle.estimate(q, k, v, mu, np.zeros(0, np.int32), 4, 16, 1, 16)
    assert np.allclose(out_t, _softmax_attention_torch(q, k, v, T), rtol=0, atol=1e-13)
    assert not oracle.estimate(q, k, v, mu, np.zeros(0, np.int32), 4, 16, 0, 0).any()


def test_estimator_converges_in_L():
    Ls = [4, 16, 64, 256]
    errs = {L: [] for L in Ls}
    frac = {L: [] for L in Ls}
    for s in range(12):
        k, v, q = _tiny_inputs(s)
        o = _softmax_attention_torch(q, k, v)
        K, Lm = 4, Ls[-1]
        W = oracle.hyperplanes(seed=1000 + s, R=K * Lm, d=128)
        mu = oracle.mean(k)
        codes, _ = oracle.encode_keys_parallel(k, W, K, Lm, mu)
        qc, _ = oracle.encode(q, W, K, Lm)
        prev = None
        for L in Ls:
            # W of L tables is the row prefix of W of Lm tables
            counts = oracle.collision_counts(codes[:L], qc[:L])
            S = oracle.select(counts, 1, 16)
            if prev is not None:
                assert set(prev) <= set(S)          # nested tables => nested sets
            prev = S
            oh = oracle.estimate(q, k, v, mu, S, K, L, 1, 16)
            errs[L].append(np.linalg.norm(oh - o) / np.linalg.norm(o))
            frac[L].append(len(S) / (1024 - 17))
    means = [np.mean(errs[L]) for L in Ls]
    for a, b in zip(means, means[1:]):
        assert b < 0.6 * a, means
    assert np.mean(frac[256]) > 0.99
    assert means[-1] < 0.05


def test_horvitz_thompson_inclusion_and_sums():
    """Set-inclusion semantics: E[1{i in S}] = u_i, and the estimator's two sums
    sum_S w_i v_i / u_i and sum_S w_i / u_i are unbiased for the sums over all
    keys outside T (w_i = exp(q.k_i/sqrt(d))).

    The sums are read back out of ``estimate`` itself: the one exact key (the
    sink, in T) carries value e_0 and every other key has 0 in coordinate 0,
    so out[0] = w_T / (D_S + w_T) and out[1:] = N_S / (D_S + w_T)."""
    rng = np.random.default_rng(11)
    n, d, K, L = 12, 8, 2, 4
    k = rng.standard_normal((n, d))
    vals = rng.standard_normal((n, 3))
    q = rng.standard_normal(d)
    n_sink, n_local = 1, 0
    v = np.zeros((n, d))
    v[0, 0] = 1.0
    v[1:, 1:4] = vals[1:]
    mu = oracle.mean(k)
    x = k - mu
    uvec = np.array([oracle.u(oracle.collision_p(q, x[i]), K, L) for i in range(n)])
    wt = np.exp(k @ q / math.sqrt(d))
    R = 10000
    inc = np.zeros(n)
    num = np.zeros((R, 3))
    den = np.zeros(R)
    size = np.zeros(R)
    for s in range(R):
        W = oracle.hyperplanes(seed=9_000_000 + s, R=K * L, d=d)
        codes, _ = oracle.encode_keys(k, W, K, L, mu)
        qc, _ = oracle.encode(q, W, K, L)
        S = oracle.select(oracle.collision_counts(codes, qc), n_sink, n_local)
        inc[S] += 1
        size[s] = len(S)
        out = oracle.estimate(q, k, v, mu, S, K, L, n_sink, n_local)
        total = wt[0] / out[0]
        den[s] = total - wt[0]
        num[s] = out[1:4] * total
    mid = np.arange(n_sink, n - n_local)
    assert inc[0] == 0
    f = inc[mid] / R
    sig = np.sqrt(uvec[mid] * (1 - uvec[mid]) / R)
    assert np.all(np.abs(f - uvec[mid]) <= 4.5 * sig), (f, uvec[mid])
    assert abs(size.mean() - uvec[mid].sum()) <= 4.5 * size.std() / math.sqrt(R)
    true_num = (wt[mid, None] * vals[mid]).sum(0)
    assert np.all(np.abs(num.mean(0) - true_num) <= 4.5 * num.std(0) / math.sqrt(R)), \
        (num.mean(0), true_num)
    assert abs(den.mean() - wt[mid].sum()) <= 4.5 * den.std() / math.sqrt(R), \
        (den.mean(), wt[mid].sum())
    assert 0.02 < uvec[mid].min() and uvec[mid].max() < 0.98   # probabilities genuinely vary


def _u_closed_form(p, K, L):
    """P[Binomial(L, p^K) >= 2] in exact rationals (no oracle call)."""
    P = Fraction(p) ** K
    return float(1 - (1 - P) ** L - L * P * (1 - P) ** (L - 1))


def _mirrored_keys(rng, m, d, n_center):
    """2m keys in mirrored pairs c +- delta plus n_center copies of c: every
    value is a multiple of 2^-10 below 1 in magnitude, so the fp64 sums are
    exact and the mean is exactly c."""
    c = rng.choice([-0.5, 0.5], size=d)
    delta = np.round(rng.uniform(-0.49, 0.49, size=(m, d)) * 1024) / 1024
    k = np.concatenate([c + delta, c - delta, np.tile(c, (n_center, 1))])
    return k[rng.permutation(len(k))], c


def test_zero_length_vectors_are_included_with_u_of_one_half():
    """The zero-length reading (page "MagicPIG: don't pick the tallest",
    section 5: zero-length vectors need a rule): a vector of length 0 has
    every projection exactly 0, so with sign(0) = 0 its code is 0 in every
    table; a random hyperplane puts a fixed other vector on either side with
    probability 1/2, so one table matches with probability 2^-K and the pair
    collides in >= 2 of L tables with probability u(p = 1/2).  The oracle's
    cosine-0 rule (p = 1/2) is therefore the true inclusion probability, for a
    centered key equal to the mean and for a zero query alike."""
    rng = np.random.default_rng(21)
    d, K, L, R = 16, 2, 6, 4000
    k, c = _mirrored_keys(rng, 4, d, 1)
    mu = oracle.mean(k)
    assert np.array_equal(mu, c)
    i0 = int(np.nonzero((k == c).all(1))[0][0])
    q = rng.standard_normal(d)
    zero = np.zeros(d)
    u_half = _u_closed_form(Fraction(1, 2), K, L)
    assert oracle.collision_p(q, k[i0] - mu) == 0.5
    assert oracle.collision_p(zero, k[3] - mu) == 0.5
    assert oracle.u(0.5, K, L) == pytest.approx(u_half, rel=1e-13)
    j0 = (i0 + 3) % len(k)                     # a key of nonzero centered length
    hit_key = hit_q = 0
    for s in range(R):
        W = oracle.hyperplanes(seed=7_000_000 + s, R=K * L, d=d)
        codes, _ = oracle.encode_keys(k, W, K, L, mu)
        assert not codes[:, i0].any()          # the zero vector's code is 0 everywhere
        qc, _ = oracle.encode(q, W, K, L)
        hit_key += int(np.count_nonzero(codes[:, i0] == qc) >= 2)
        qz, _ = oracle.encode(zero, W, K, L)
        assert not qz.any()
        hit_q += int(np.count_nonzero(codes[:, j0] == qz) >= 2)
    tol = 5 * math.sqrt(u_half * (1 - u_half) / R)
    assert abs(hit_key / R - u_half) <= tol, (hit_key / R, u_half)
    assert abs(hit_q / R - u_half) <= tol, (hit_q / R, u_half)


def test_zero_query_estimate_is_the_closed_form():
    """q = 0: every score is 0 and every sampled key has p = 1/2, so the
    estimate is (sum_S v_i / u(1/2) + sum_T v_i) / (|S| / u(1/2) + |T|)."""
    rng = np.random.default_rng(5)
    n, d, K, L = 40, 128, 3, 10
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    S = np.array([2, 5, 6, 11, 30], dtype=np.int32)
    T = [0, 1] + list(range(n - 4, n))
    u = _u_closed_form(Fraction(1, 2), K, L)
    ref = (v[S].sum(0) / u + v[T].sum(0)) / (len(S) / u + len(T))
    out = oracle.estimate(np.zeros(d), k, v, oracle.mean(k), S, K, L, 2, 4)
    assert np.max(np.abs(out - ref)) <= 1e-13 * np.max(np.abs(ref))
    # a centered key equal to the mean gets p = 1/2 as well: with q != 0 its
    # weight is exp(q.k/sqrt(d)) / u(1/2)
    k2, c = _mirrored_keys(rng, 6, d, 1)
    i0 = int(np.nonzero((k2 == c).all(1))[0][0])
    v2 = rng.standard_normal((len(k2), d))
    q = rng.standard_normal(d)
    j = (i0 + 1) % len(k2)
    mu2 = oracle.mean(k2)
    uj = _u_closed_form(Fraction(1) - Fraction(math.acos(
        float(np.dot(q, k2[j] - mu2) / np.linalg.norm(q) / np.linalg.norm(k2[j] - mu2))) / math.pi),
        K, L)
    z = np.array([q @ k2[i0] / math.sqrt(d) - math.log(u), q @ k2[j] / math.sqrt(d) - math.log(uj)])
    w = np.exp(z - z.max())
    ref2 = (w[0] * v2[i0] + w[1] * v2[j]) / w.sum()
    out2 = oracle.estimate(q, k2, v2, mu2, np.array(sorted([i0, j]), np.int32), K, L, 0, 0)
    assert np.max(np.abs(out2 - ref2)) <= 1e-9 * np.max(np.abs(ref2))


def test_centering_is_score_invariant_and_needed():
    k, v, q = _tiny_inputs(5)
    K, L = 4, 16
    W = oracle.hyperplanes(seed=5, R=K * L, d=128)
    mu = oracle.mean(k)
    codes, _ = oracle.encode_keys(k, W, K, L, mu)
    qc, _ = oracle.encode(q, W, K, L)
    S = oracle.select(oracle.collision_counts(codes, qc), 1, 16)
    a = oracle.estimate(q, k, v, mu, S, K, L, 1, 16)
    b = oracle.estimate(q, k, v, mu, S, K, L, 1, 16, flags=oracle.SCORE_CENTERED)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    assert len(S) / 1007 > 0.15
    # without centering the keys sit in a cone facing away from q: almost no
    # key collides in two tables
    fr = []
    for s in range(4):
        k, v, q = _tiny_inputs(20 + s)
        W = oracle.hyperplanes(seed=20 + s, R=K * L, d=128)
        codes, _ = oracle.encode_keys(k, W, K, L, None)
        qc, _ = oracle.encode(q, W, K, L)
        fr.append(len(oracle.select(oracle.collision_counts(codes, qc), 1, 16)) / 1007)
    assert np.mean(fr) < 1e-3


def test_frozen_mean_append_equals_full_build_when_the_mean_holds():
    """Reading for a growing index (the pages fix the mean only for a static
    set of keys): keys that arrive later are centered by the mean of the keys
    the index was built on.  When the new keys come in pairs mu0 + e, mu0 - e,
    the mean of all keys is still mu0, so the grown index must be the index a
    full build over all keys gives: same codes, counts, sets and estimate."""
    k, v, q = _tiny_inputs(31)
    K, L = 5, 24
    W = oracle.hyperplanes(seed=31, R=K * L, d=128)
    n0 = 600
    mu0 = oracle.mean(k[:n0])
    rng = np.random.default_rng(31)
    e = rng.standard_normal((150, 128)) * 0.3
    k_new = np.concatenate([mu0 + e, mu0 - e])            # mean exactly mu0 in fp64 sums
    k_all = np.concatenate([k[:n0], k_new])
    v_all = np.concatenate([v[:n0], rng.standard_normal((300, 128))])
    mu_all = oracle.mean(k_all)
    assert np.max(np.abs(mu_all - mu0)) <= 1e-12
    grown = np.concatenate([oracle.encode_keys(k[:n0], W, K, L, mu0)[0],
                            oracle.encode_keys(k_new, W, K, L, mu0)[0]], axis=1)
    full, _ = oracle.encode_keys(k_all, W, K, L, mu_all)
    differ = grown != full
    # codes may differ only where a projection sits in the 1e-5 band
    for l, i in zip(*np.nonzero(differ)):
        _, band = oracle.encode(k_all[i] - mu0, W, K, L)
        assert band[l * K:(l + 1) * K].any()
    assert differ.sum() <= 1
    qc, _ = oracle.encode(q, W, K, L)
    cg, cf = oracle.collision_counts(grown, qc), oracle.collision_counts(full, qc)
    S = oracle.select(cg, 1, 16)
    if not differ.any():
        assert np.array_equal(cg, cf)
        a = oracle.estimate(q, k_all, v_all, mu0, S, K, L, 1, 16)
        b = oracle.estimate(q, k_all, v_all, mu_all, oracle.select(cf, 1, 16), K, L, 1, 16)
        assert np.max(np.abs(a - b)) <= 1e-9 * np.max(np.abs(b))
    # and a key appended again is coded exactly like its first copy
    again = oracle.encode_keys(k[:40], W, K, L, mu0)[0]
    assert np.array_equal(again, grown[:, :40])


def test_mean_matches_exact_column_sums():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((3000, 7)) * 5 + 1
    mu = oracle.mean(k)
    for c in range(7):
        assert mu[c] == pytest.approx(math.fsum(k[:, c].tolist()) / 3000, rel=1e-14, abs=1e-15)


@pytest.mark.slow
def test_band_fraction_matches_closed_form():
    """Fraction of |w.x| < 1e-5 |w||x| over random hyperplanes: P(|cos| < eps)
    for a uniformly random direction in d dimensions = I_{eps^2}(1/2, (d-1)/2)."""
    from scipy.special import betainc
    cfg = synth.CONFIGS["llama8b_16k"]
    inp = synth.cone_inputs(B=1, H_q=4, H_kv=1, n=4096, d=128, dtype=torch.bfloat16, seeds=[42])
    k = inp["k"][0, 0].double().numpy()
    W = oracle.hyperplanes(seed=42, R=cfg.K * cfg.L, d=128)
    mu = oracle.mean(k)
    _, nb = oracle.encode_keys_parallel(k, W, cfg.K, cfg.L, mu)
    N = k.shape[0] * cfg.K * cfg.L
    p = betainc(0.5, 63.5, 1e-10)
    assert p == pytest.approx(8.97e-5, rel=2e-3)
    assert abs(nb - N * p) <= 3 * math.sqrt(N * p), (nb, N * p)


# ---------------------------------------------------------------- integer steps
@pytest.mark.parametrize("n_sink,n_local", [(0, 0), (4, 64), (1, 16), (300, 250), (600, 0),
                                            (0, 900), (10, 10)])
def test_counts_and_select_brute_force(n_sink, n_local):
    rng = np.random.default_rng(n_sink * 1000 + n_local)
    L, n = 7, 500
    codes = rng.integers(0, 4, size=(L, n)).astype(np.uint16)
    qc = rng.integers(0, 4, size=L).astype(np.uint16)
    counts = oracle.collision_counts(codes, qc)
    ref = np.array([sum(int(codes[l, i] == qc[l]) for l in range(L)) for i in range(n)])
    assert np.array_equal(counts, ref)
    S = oracle.select(counts, n_sink, n_local)
    refS = [i for i in range(n) if ref[i] >= 2 and not (i < n_sink or i >= n - n_local)]
    assert S.tolist() == refS


def test_estimate_rejects_out_of_range_index():
    k, v, q = _tiny_inputs(1)
    with pytest.raises(ValueError):
        oracle.estimate(q, k, v, oracle.mean(k), np.array([5, 4000], np.int32), 4, 16, 1, 16)


# ---- inner-product-to-cosine augmentation ([P2] method details) ----
def test_augmentation_with_keys_on_a_sphere_changes_nothing():
    """Keys all at distance r from their mean lift with a zero extra
    coordinate: the lifted codes are the plain codes and the lifted cosine is
    the plain one, so codes, sets and the estimate agree exactly."""
    rng = np.random.default_rng(41)
    K, L, n = 4, 16, 700
    mu = rng.standard_normal(128) * 0.5
    x = rng.standard_normal((n // 2, 128))
    x *= 3.0 / np.linalg.norm(x, axis=1, keepdims=True)
    k = mu + np.concatenate([x, -x])                   # pairs +x, -x: the mean is mu
    mu = oracle.mean(k)
    v = rng.standard_normal((n, 128))
    q = rng.standard_normal(128)
    W = oracle.hyperplanes(41, K * L, 128)
    w = oracle.hyperplane_extra(41, K * L, 128)
    r = oracle.aug_radius(k, mu)
    assert r == pytest.approx(3.0, rel=1e-9)
    plain, _ = oracle.encode_keys(k, W, K, L, mu)
    lifted, _ = oracle.encode_keys_aug(k, W, w, K, L, mu, r)
    # the extra coordinate is sqrt(r^2 - |x|^2) ~ 1e-7 r here; a flip needs a
    # projection within that of zero
    assert (plain != lifted).sum() <= 2
    qc, _ = oracle.encode(q, W, K, L)
    S = oracle.select(oracle.collision_counts(plain, qc), 1, 16)
    a = oracle.estimate(q, k, v, mu, S, K, L, 1, 16)
    b = oracle.estimate(q, k, v, mu, S, K, L, 1, 16, aug_r=r)
    assert np.max(np.abs(a - b)) <= 1e-6 * np.max(np.abs(a))


def test_augmented_agreement_rate_is_one_minus_lifted_angle_over_pi():
    """Monte Carlo over 20000 one-bit tables: a key of norm r/3 agrees with the
    query in a fraction 1 - theta/pi of them, theta the angle of the lifted
    pair (cos = q.x / (|q| r)), not of the plain pair."""
    rng = np.random.default_rng(42)
    d, L = 128, 20000
    q = rng.standard_normal(d)
    q /= np.linalg.norm(q)
    e = rng.standard_normal(d)
    e -= (e @ q) * q
    e /= np.linalg.norm(e)
    r = 3.0
    x_small = (0.9 * q + math.sqrt(1 - 0.81) * e) * (r / 3)    # plain cos 0.9, lifted 0.3
    x_far = -q * r                                             # sets r; lifted = plain
    keys = np.stack([x_small, x_far])
    W = oracle.hyperplanes(42, L, d)
    w = oracle.hyperplane_extra(42, L, d)
    assert oracle.aug_radius(keys, None) == pytest.approx(r)
    codes, _ = oracle.encode_keys_aug(keys, W, w, 1, L, None, r)
    qc, _ = oracle.encode(q, W, 1, L)
    agree = (codes[:, 0] == qc).mean()
    lifted = 1 - math.acos(0.3) / math.pi
    plain = 1 - math.acos(0.9) / math.pi
    sigma = math.sqrt(lifted * (1 - lifted) / L)
    assert abs(agree - lifted) < 5 * sigma, (agree, lifted, plain)
    assert abs(agree - plain) > 20 * sigma
    assert (codes[:, 1] == qc).mean() == pytest.approx(0.0, abs=1e-12)   # antiparallel


def test_augmented_p_orders_keys_by_inner_product():
    """The point of the lift: p_i grows with q.x_i whatever |x_i| is."""
    rng = np.random.default_rng(43)
    k = rng.standard_normal((300, 128)) * rng.uniform(0.2, 3.0, (300, 1))
    q = rng.standard_normal(128)
    mu = oracle.mean(k)
    r = oracle.aug_radius(k, mu)
    x = k - mu
    lifted_k = np.concatenate([x, np.sqrt(np.maximum(r * r - (x * x).sum(1), 0))[:, None]], 1)
    lifted_q = np.concatenate([q, [0.0]])
    p = np.array([oracle.collision_p(lifted_q, lk) for lk in lifted_k])
    order = np.argsort(x @ q)
    assert np.all(np.diff(p[order]) >= -1e-12)
    p_plain = np.array([oracle.collision_p(q, xi) for xi in x])
    assert not np.all(np.diff(p_plain[order]) >= -1e-12)     # the plain cosine does not


def test_augmented_estimate_weighs_equal_inner_products_equally():
    """Two sampled keys with the same q.k and q.(k - mu) but different norms:
    under the lift their u are equal, so the estimate is the plain mean of
    their values; under the plain cosine it is not."""
    rng = np.random.default_rng(44)
    d = 128
    q = rng.standard_normal(d)
    qh = q / np.linalg.norm(q)
    e1, e2 = rng.standard_normal(d), rng.standard_normal(d)
    for e in (e1, e2):
        e -= (e @ qh) * qh
        e /= np.linalg.norm(e)
    mu = rng.standard_normal(d) * 0.1
    x1 = 0.8 * qh + 0.3 * e1
    x2 = 0.8 * qh + 1.7 * e2
    x3 = -2.5 * qh                                         # only sets the radius
    k = mu + np.stack([x1, x2, x3])
    v = rng.standard_normal((3, d))
    r = oracle.aug_radius(k, mu)
    S = np.array([0, 1], dtype=np.int32)
    lifted = oracle.estimate(q, k, v, mu, S, 6, 30, 0, 0, aug_r=r)
    assert np.max(np.abs(lifted - (v[0] + v[1]) / 2)) <= 1e-12
    plain = oracle.estimate(q, k, v, mu, S, 6, 30, 0, 0)
    assert np.max(np.abs(plain - (v[0] + v[1]) / 2)) > 1e-3
