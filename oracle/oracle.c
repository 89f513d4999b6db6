/*
 * oracle.c -- plain, slow fp64 CPU reference of MagicPIG's decode-time
 * attention estimator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark load this library.  It shares no code
 * with the HIP path (no headers, no helpers, no tables) and the HIP path never
 * calls it.
 *
 * Sources (the pages this follows):
 *   [P1] "MagicPIG: don't pick the tallest" (borzov.ca), sections 5 "A hash
 *        that knows its odds" and 6 "The bill".
 *   [P2] "MagicPIG: LSH Sampling for Efficient LLM Generation" (papercache.org
 *        summary of arXiv 2410.16179): background section (SimHash),
 *        method-details section (self-normalised importance sampling, the
 *        collision probability u_i, centering, the algorithm's steps) and the
 *        system co-design section (exact sink/local tokens, merged outputs).
 *
 * All arithmetic is IEEE fp64 (build without -ffast-math).  Inputs given as
 * bf16/fp32 are converted to fp64 exactly by the caller.
 *
 * Readings where the pages are silent:
 *   - hyperplanes: element e of the row-major [R][d] matrix W is a standard
 *     normal made by the Box-Muller transform (Box & Muller 1958) from the
 *     outputs 2e+1 and 2e+2 of SplitMix64 (Steele, Lea & Flood, OOPSLA 2014)
 *     seeded with `seed`, then rounded to fp32; row j = l*K + b is bit b of
 *     table l, so a smaller L uses a row prefix of a larger L's W;
 *   - the sign bit is 1 iff the projection is > 0 (strictly), and the K bits
 *     of a table are packed least-significant-bit first into a uint16 code;
 *   - only keys are centered (by the mean of all n keys); queries are hashed raw;
 *   - the cosine inside p_i uses the centered key (the vector that was hashed),
 *     scores use the raw key;
 *   - the exact set T is [0, n_sink) u [n - n_local, n); S excludes T;
 *   - a zero-length query or centered key gives cosine 0.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

/* ------------------------------------------------------------------------ */
/* Hyperplanes W ~ N(0, 1)                                                   */
/* ------------------------------------------------------------------------ */

/* k-th output (k >= 1) of SplitMix64 started at `seed`: the state after k
 * increments of the golden-ratio constant, passed through the finaliser. */
uint64_t orc_splitmix64(uint64_t seed, uint64_t k)
{
    uint64_t z = seed + k * ORC_GOLDEN_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Standard normal number e of the stream (Box-Muller, cosine branch). */
double orc_gauss(uint64_t seed, uint64_t e)
{
    uint64_t z1 = orc_splitmix64(seed, 2 * e + 1);
    uint64_t z2 = orc_splitmix64(seed, 2 * e + 2);
    double u1 = ((double)(z1 >> 11) + 1.0) * 0x1.0p-53;  /* (0, 1] */
    double u2 = (double)(z2 >> 11) * 0x1.0p-53;          /* [0, 1) */
    return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

/* Rows [row0, row0 + nrows) of W (d columns), rounded to fp32. */
void orc_hyperplanes(uint64_t seed, int64_t row0, int64_t nrows, int d, float *W)
{
    for (int64_t r = 0; r < nrows; ++r)
        for (int c = 0; c < d; ++c) {
            uint64_t e = (uint64_t)(row0 + r) * (uint64_t)d + (uint64_t)c;
            W[r * d + c] = (float)orc_gauss(seed, e);
        }
}

/* ------------------------------------------------------------------------ */
/* Centering: mu = (1/n) sum_i k_i  ([P2] method details, centering;         */
/* [P1] section 5: every score shifts by q.mu, which softmax ignores)        */
/* ------------------------------------------------------------------------ */

void orc_mean(const double *keys, int64_t n, int d, double *mu)
{
    for (int c = 0; c < d; ++c) mu[c] = 0.0;
    for (int64_t i = 0; i < n; ++i)
        for (int c = 0; c < d; ++c) mu[c] += keys[i * d + c];
    for (int c = 0; c < d; ++c) mu[c] /= (double)n;
}

/* ------------------------------------------------------------------------ */
/* SimHash ([P2] background: h(x) = sign(w^T x), agreement 1 - theta/pi;     */
/* [P2] method details: K*L random vectors, K sign bits per table)          */
/* ------------------------------------------------------------------------ */

/* bits[j] = [w_j . x > 0]; band[j] (optional) = [|w_j . x| < 1e-5 |w_j||x|]. */
void orc_project_signs(const double *x, int d, const float *W, int64_t R,
                       uint8_t *bits, uint8_t *band)
{
    double xx = 0.0;
    for (int c = 0; c < d; ++c) xx += x[c] * x[c];
    double xn = sqrt(xx);
    for (int64_t j = 0; j < R; ++j) {
        const float *w = W + j * d;
        double proj = 0.0, ww = 0.0;
        for (int c = 0; c < d; ++c) {
            proj += (double)w[c] * x[c];
            ww += (double)w[c] * (double)w[c];
        }
        bits[j] = proj > 0.0 ? 1 : 0;
        if (band) band[j] = fabs(proj) < 1e-5 * sqrt(ww) * xn ? 1 : 0;
    }
}

/* code[l] = sum_{b<K} bits[l*K + b] << b. */
void orc_pack_codes(const uint8_t *bits, int K, int L, uint16_t *code)
{
    for (int l = 0; l < L; ++l) {
        unsigned v = 0;
        for (int b = 0; b < K; ++b) v |= (unsigned)bits[l * K + b] << b;
        code[l] = (uint16_t)v;
    }
}

/* Codes of one vector; optional band flags [K*L]; returns the band count. */
int64_t orc_encode(const double *x, int d, const float *W, int K, int L,
                   uint16_t *code, uint8_t *band)
{
    int64_t R = (int64_t)K * L;
    uint8_t *bits = (uint8_t *)malloc((size_t)(R > 0 ? R : 1));
    uint8_t *bd = band ? band : (uint8_t *)malloc((size_t)(R > 0 ? R : 1));
    orc_project_signs(x, d, W, R, bits, bd);
    orc_pack_codes(bits, K, L, code);
    int64_t nb = 0;
    for (int64_t j = 0; j < R; ++j) nb += bd[j];
    free(bits);
    if (!band) free(bd);
    return nb;
}

/* Table-major key codes codes[l*n + i] of x_i = k_i - mu (mu == NULL: raw
 * keys, the no-centering ablation).  Returns the number of band bits. */
int64_t orc_encode_keys(const double *keys, int64_t n, int d, const double *mu,
                        const float *W, int K, int L, uint16_t *codes)
{
    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    uint16_t *code = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(L > 0 ? L : 1));
    int64_t nb = 0;
    for (int64_t i = 0; i < n; ++i) {
        for (int c = 0; c < d; ++c) x[c] = keys[i * d + c] - (mu ? mu[c] : 0.0);
        nb += orc_encode(x, d, W, K, L, code, NULL);
        for (int l = 0; l < L; ++l) codes[(int64_t)l * n + i] = code[l];
    }
    free(x);
    free(code);
    return nb;
}

/* orc_encode_keys plus, per table and key, the mask of the code's bits that
 * lie in the band |w_j . x| < 1e-5 |w_j||x| (bit b of band[l*n + i] belongs
 * to hyperplane l*K + b): a sign that close to 0 depends on the order in
 * which the projection is summed, so a comparison may accept either value
 * there.  The projections, norms and band test are those of
 * orc_project_signs, with |w_j| (which does not depend on the key) computed
 * once per hyperplane.  Returns the band count. */
int64_t orc_encode_keys_band(const double *keys, int64_t n, int d, const double *mu,
                             const float *W, int K, int L, uint16_t *codes, uint16_t *band)
{
    int64_t R = (int64_t)K * L;
    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    double *wn = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    for (int64_t j = 0; j < R; ++j) {
        double ww = 0.0;
        for (int c = 0; c < d; ++c) ww += (double)W[j * d + c] * (double)W[j * d + c];
        wn[j] = sqrt(ww);
    }
    int64_t nb = 0;
    for (int64_t i = 0; i < n; ++i) {
        double xx = 0.0;
        for (int c = 0; c < d; ++c) {
            x[c] = keys[i * d + c] - (mu ? mu[c] : 0.0);
            xx += x[c] * x[c];
        }
        double xn = sqrt(xx);
        for (int l = 0; l < L; ++l) {
            unsigned code = 0, m = 0;
            for (int b = 0; b < K; ++b) {
                const float *w = W + ((int64_t)l * K + b) * d;
                double proj = 0.0;
                for (int c = 0; c < d; ++c) proj += (double)w[c] * x[c];
                code |= (unsigned)(proj > 0.0) << b;
                m |= (unsigned)(fabs(proj) < 1e-5 * wn[(int64_t)l * K + b] * xn) << b;
            }
            codes[(int64_t)l * n + i] = (uint16_t)code;
            band[(int64_t)l * n + i] = (uint16_t)m;
            nb += __builtin_popcount(m);
        }
    }
    free(x);
    free(wn);
    return nb;
}

/* ------------------------------------------------------------------------ */
/* Inner-product-to-cosine augmentation ([P2] method details, variance        */
/* reduction with LSH): with r the largest key norm, every key is lifted to   */
/* [x, sqrt(r^2 - |x|^2)] (norm r) and the query to [q, 0], so the cosine of  */
/* the lifted pair is q.x / (|q| r), monotone in q.x.  Here x = k - mu, the  */
/* centered key (centering is applied first, as for the plain path).  The     */
/* extra hyperplane coordinate j is normal number R*d + j of the same stream  */
/* (R = K*L): the lifted hyperplane j is [W_j, w_j].                          */
/* ------------------------------------------------------------------------ */

/* r = max_i |k_i - mu| (mu == NULL: raw keys). */
double orc_aug_radius(const double *keys, int64_t n, int d, const double *mu)
{
    double r2 = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) {
            double x = keys[i * d + c] - (mu ? mu[c] : 0.0);
            s += x * x;
        }
        if (s > r2) r2 = s;
    }
    return sqrt(r2);
}

/* The extra coordinate of the R lifted hyperplanes, rounded to fp32. */
void orc_hyperplane_extra(uint64_t seed, int64_t R, int d, float *w)
{
    for (int64_t j = 0; j < R; ++j) w[j] = (float)orc_gauss(seed, (uint64_t)(R * d + j));
}

/* Table-major codes of the lifted keys [k_i - mu, sqrt(r^2 - |k_i - mu|^2)]
 * against the lifted hyperplanes [W_j, w_j]; returns the band count (the band
 * taken on the lifted vectors). */
int64_t orc_encode_keys_aug(const double *keys, int64_t n, int d, const double *mu,
                            const float *W, const float *w, double r, int K, int L,
                            uint16_t *codes)
{
    int64_t R = (int64_t)K * L;
    float *Wl = (float *)malloc(sizeof(float) * (size_t)((R > 0 ? R : 1) * (d + 1)));
    for (int64_t j = 0; j < R; ++j) {
        for (int c = 0; c < d; ++c) Wl[j * (d + 1) + c] = W[j * d + c];
        Wl[j * (d + 1) + d] = w[j];
    }
    double *x = (double *)malloc(sizeof(double) * (size_t)(d + 1));
    uint16_t *code = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(L > 0 ? L : 1));
    int64_t nb = 0;
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int c = 0; c < d; ++c) {
            x[c] = keys[i * d + c] - (mu ? mu[c] : 0.0);
            s += x[c] * x[c];
        }
        x[d] = r * r > s ? sqrt(r * r - s) : 0.0;
        nb += orc_encode(x, d + 1, Wl, K, L, code, NULL);
        for (int l = 0; l < L; ++l) codes[(int64_t)l * n + i] = code[l];
    }
    free(Wl);
    free(x);
    free(code);
    return nb;
}

/* ------------------------------------------------------------------------ */
/* Sampling rule ([P2] method details; [P1] section 5): a key is sampled     */
/* iff it shares the query's bucket in at least two of the L tables, and the */
/* sampled set S leaves out the exact (sink + local) set T.                  */
/* ------------------------------------------------------------------------ */

/* counts[i] = #{l : codes[l][i] == qcode[l]} */
void orc_collision_counts(const uint16_t *codes, int64_t n, int L,
                          const uint16_t *qcode, int32_t *counts)
{
    for (int64_t i = 0; i < n; ++i) {
        int32_t c = 0;
        for (int l = 0; l < L; ++l)
            if (codes[(int64_t)l * n + i] == qcode[l]) ++c;
        counts[i] = c;
    }
}

int orc_in_exact_set(int64_t i, int64_t n, int64_t n_sink, int64_t n_local)
{
    return i < n_sink || i >= n - n_local;
}

/* S in ascending order; returns |S|. */
int64_t orc_select(const int32_t *counts, int64_t n, int64_t n_sink,
                   int64_t n_local, int32_t *idx)
{
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i)
        if (counts[i] >= 2 && !orc_in_exact_set(i, n, n_sink, n_local))
            idx[m++] = (int32_t)i;
    return m;
}

/* ------------------------------------------------------------------------ */
/* Collision probability ([P2] quick read and method details; [P1] sec. 5):  */
/*   p = 1 - arccos(cos)/pi is the chance that one bit agrees,               */
/*   P = p^K that a whole table agrees (independent bits),                   */
/*   u = P[at least 2 of L independent tables agree]                         */
/*     = 1 - (1-P)^L - L P (1-P)^(L-1).                                      */
/* Where L*P is small the two subtractions cancel ([P1] section 5 asks for    */
/* stable probability arithmetic), so there u is summed as the binomial tail */
/* sum_{j>=2} C(L,j) P^j (1-P)^(L-j), in logs.                               */
/* ------------------------------------------------------------------------ */

double orc_log_u(double p, int K, int L)
{
    if (L < 2) return -INFINITY;
    double P = pow(p, (double)K);       /* pow(x, 0) == 1: K = 0 samples all */
    if (P >= 1.0) return 0.0;
    if (P <= 0.0) return -INFINITY;
    double a = log1p(-P);               /* log(1 - P) */
    if ((double)L * P > 0.05) {
        double u = 1.0 - exp((double)L * a) - (double)L * P * exp((double)(L - 1) * a);
        return log(u);
    }
    /* tail = 1 + sum_{j>=3} prod_{i=2}^{j-1} r_i, r_i = (L-i)/(i+1) * P/(1-P) */
    double ratio = P / (1.0 - P);
    double term = 1.0, tail = 1.0;
    for (int j = 2; j < L; ++j) {
        term *= (double)(L - j) / (double)(j + 1) * ratio;
        tail += term;
        if (term < 1e-18 * tail) break;
    }
    return log(0.5 * (double)L * (double)(L - 1)) + 2.0 * log(P)
           + (double)(L - 2) * a + log(tail);
}

double orc_u(double p, int K, int L)
{
    return exp(orc_log_u(p, K, L));
}

/* p = 1 - arccos(cos(a, b))/pi; cosine 0 when either vector has length 0. */
double orc_collision_p(const double *a, const double *b, int d)
{
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int c = 0; c < d; ++c) {
        ab += a[c] * b[c];
        aa += a[c] * a[c];
        bb += b[c] * b[c];
    }
    double cs = (aa > 0.0 && bb > 0.0) ? ab / (sqrt(aa) * sqrt(bb)) : 0.0;
    if (cs > 1.0) cs = 1.0;
    if (cs < -1.0) cs = -1.0;
    return 1.0 - acos(cs) / M_PI;
}

/* ------------------------------------------------------------------------ */
/* Estimator ([P2] method details: self-normalised importance sampling over  */
/* S with weights exp(q.k/sqrt(d)) / u_i; the algorithm's last step takes    */
/* one softmax over [w_S, w_T]/sqrt(d) - log[u, 1] against [V_S, V_T]).      */
/* ------------------------------------------------------------------------ */

#define ORC_SCORE_CENTERED 1   /* scores use q.(k - mu): centering-invariance check */
#define ORC_CONST_LOG_U    2   /* every key of S gets log u = const_log_u            */
#define ORC_AUGMENTED      4   /* p_i from the lifted pair [q, 0], [x_i, sqrt(r^2 - |x_i|^2)] */

/* out[d] = sum_{i in S u T} e^{z_i - M} v_i / sum e^{z_i - M}, where
 * z_i = scale q.k_i - log u_i on S and scale q.k_i on T, M = max z.
 * mu == NULL: cosines against raw keys (no-centering ablation).
 * Returns 0, or -1 if a key of S has u == 0 (not reachable by the sampling
 * rule in exact arithmetic), or -2 for an index out of range. */
int orc_estimate(const double *q, const double *keys, const double *values,
                 const double *mu, int64_t n, int d, int K, int L,
                 const int32_t *S, int64_t s_len, int64_t n_sink, int64_t n_local,
                 double scale, int flags, double const_log_u, double aug_r, double *out)
{
    int64_t t_lo = n_sink < n ? n_sink : n;
    int64_t t_hi = n - n_local > t_lo ? n - n_local : t_lo;   /* T = [0,t_lo) u [t_hi,n) */
    int64_t m = s_len + t_lo + (n - t_hi);
    double *z = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    int64_t *row = (int64_t *)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
    double *x = (double *)malloc(sizeof(double) * (size_t)(d + 1));
    double *ql = (double *)malloc(sizeof(double) * (size_t)(d + 1));
    int rc = 0;
    int64_t j = 0;
    for (int c = 0; c < d; ++c) ql[c] = q[c];
    ql[d] = 0.0;

    for (int64_t s = 0; s < s_len; ++s) {
        int64_t i = S[s];
        if (i < 0 || i >= n) { rc = -2; goto done; }
        const double *k = keys + i * d;
        double qk = 0.0;
        for (int c = 0; c < d; ++c) {
            x[c] = k[c] - (mu ? mu[c] : 0.0);
            qk += q[c] * ((flags & ORC_SCORE_CENTERED) ? x[c] : k[c]);
        }
        double lu;
        if (flags & ORC_CONST_LOG_U) {
            lu = const_log_u;
        } else if (flags & ORC_AUGMENTED) {
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += x[c] * x[c];
            x[d] = aug_r * aug_r > s ? sqrt(aug_r * aug_r - s) : 0.0;
            lu = orc_log_u(orc_collision_p(ql, x, d + 1), K, L);
            if (!(lu > -INFINITY)) { rc = -1; goto done; }
        } else {
            lu = orc_log_u(orc_collision_p(q, x, d), K, L);
            if (!(lu > -INFINITY)) { rc = -1; goto done; }
        }
        z[j] = scale * qk - lu;
        row[j] = i;
        ++j;
    }
    for (int64_t i = 0; i < n; ++i) {
        if (!orc_in_exact_set(i, n, n_sink, n_local)) continue;
        const double *k = keys + i * d;
        double qk = 0.0;
        for (int c = 0; c < d; ++c)
            qk += q[c] * ((flags & ORC_SCORE_CENTERED) ? k[c] - (mu ? mu[c] : 0.0) : k[c]);
        z[j] = scale * qk;
        row[j] = i;
        ++j;
    }

    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (j == 0) goto done;                  /* S u T empty: output 0 */
    {
        double M = -INFINITY;
        for (int64_t t = 0; t < j; ++t) if (z[t] > M) M = z[t];
        double den = 0.0;
        for (int64_t t = 0; t < j; ++t) {
            double e = exp(z[t] - M);
            den += e;
            const double *v = values + row[t] * d;
            for (int c = 0; c < d; ++c) out[c] += e * v[c];
        }
        for (int c = 0; c < d; ++c) out[c] /= den;
    }
done:
    free(z);
    free(row);
    free(x);
    free(ql);
    return rc;
}
