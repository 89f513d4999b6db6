// gather_common.h -- device code shared by the two decode paths of
// decode.hip (code scan) and tables.hip (bucketed tables): row loads, the
// estimator's log u, cross-lane reductions, the ascending compaction of a
// chunk's sampled and exact keys, and the gather-SNIS rounds that turn a
// chunk's list into its partial softmax (page "MagicPIG: LSH Sampling for
// Efficient LLM Generation", algorithm steps: inner products, collision and
// sampling probabilities, softmax over [w_S, w_T]/sqrt(d) - log[u, 1]).
#pragma once

#include "mp_internal.h"

namespace mp {
namespace {

constexpr int kPart = kD + 2;     // partial softmax: m, l, acc[128]
#ifndef MP_ROWS_PER_GROUP
#define MP_ROWS_PER_GROUP 4
#endif
constexpr int kRowsPerGroup = MP_ROWS_PER_GROUP;  // listed rows a 16-lane group holds per round
constexpr int kRound = 16 * kRowsPerGroup;
// c2 takes a round's rows one per lane of a wave.
static_assert(kRound <= 64, "a gather round holds at most 64 rows (4 per 16-lane group)");
// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a K or V row: raw 16-byte words, then fp32.
template <typename T> struct Row8;
template <> struct Row8<float> {
    static constexpr int kLoads = 2;
    struct raw { u32x4 w[2]; };
    static __device__ __forceinline__ raw load_raw(const float *p)
    {
        return raw{{*reinterpret_cast<const u32x4 *>(p), *reinterpret_cast<const u32x4 *>(p + 4)}};
    }
    static __device__ __forceinline__ void convert(const raw &r, float (&o)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[j] = __uint_as_float(r.w[0][j]);
            o[4 + j] = __uint_as_float(r.w[1][j]);
        }
    }
    static __device__ __forceinline__ void store_raw(float *p, const raw &r)
    {
        reinterpret_cast<u32x4 *>(p)[0] = r.w[0];
        reinterpret_cast<u32x4 *>(p)[1] = r.w[1];
    }
    static __device__ __forceinline__ void load_pair(const float *p, float &v0, float &v1)
    {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        v0 = v.x;
        v1 = v.y;
    }
};
template <> struct Row8<uint16_t> {
    static constexpr int kLoads = 1;
    struct raw { u32x4 w[1]; };
    static __device__ __forceinline__ raw load_raw(const uint16_t *p)
    {
        return raw{{*reinterpret_cast<const u32x4 *>(p)}};
    }
    static __device__ __forceinline__ void convert(const raw &r, float (&o)[8])
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = bf16_to_f32(r.w[0][j] & 0xFFFFu);
            o[2 * j + 1] = bf16_to_f32(r.w[0][j] >> 16);
        }
    }
    static __device__ __forceinline__ void store_raw(uint16_t *p, const raw &r)
    {
        *reinterpret_cast<u32x4 *>(p) = r.w[0];
    }
    static __device__ __forceinline__ void load_pair(const uint16_t *p, float &v0, float &v1)
    {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        v0 = bf16_to_f32(v & 0xFFFFu);
        v1 = bf16_to_f32(v >> 16);
    }
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---- query codes (page "MagicPIG: LSH Sampling for Efficient LLM
// Generation", background: a SimHash bit is the sign of a projection on a
// random hyperplane).  Both decode paths compute a query's projections with
// these two routines, so their codes and norms agree bit for bit.
//
// q . W_j over a group of four lanes: lane dq holds float4s 4c + dq
// (c < 8) of row W_j, so that each of the eight loads of a group reads 64
// contiguous bytes, and reads the same float4s of q (32 float4, in LDS).  Two
// FMA chains, their sum, then two shuffles over the group; all four lanes of
// the group must call it together and get the whole sum.
__device__ __forceinline__ void load_w_quarter(float4 (&wr)[8], const float *row, int dq)
{
    const float4 *w4 = reinterpret_cast<const float4 *>(row);
#pragma unroll
    for (int c = 0; c < 8; ++c) wr[c] = w4[4 * c + dq];
}

__device__ __forceinline__ float quarter_dot(const float4 (&wr)[8], const float4 *q4, int dq)
{
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
        const float4 qa = q4[4 * c + dq], qb = q4[4 * c + 4 + dq];
        a0 = fmaf(wr[c].x, qa.x, a0);
        a0 = fmaf(wr[c].y, qa.y, a0);
        a0 = fmaf(wr[c].z, qa.z, a0);
        a0 = fmaf(wr[c].w, qa.w, a0);
        a1 = fmaf(wr[c + 1].x, qb.x, a1);
        a1 = fmaf(wr[c + 1].y, qb.y, a1);
        a1 = fmaf(wr[c + 1].z, qb.z, a1);
        a1 = fmaf(wr[c + 1].w, qb.w, a1);
    }
    float sdot = a0 + a1;
    sdot += __shfl_xor(sdot, 1, 4);
    sdot += __shfl_xor(sdot, 2, 4);
    return sdot;
}

// |q| over a group of 32 lanes, lane c4 holding float4 c4 of the query; all
// 32 lanes call it together and get the norm.
__device__ __forceinline__ float norm32(float4 v)
{
    float s2 = v.x * v.x;
    s2 = fmaf(v.y, v.y, s2);
    s2 = fmaf(v.z, v.z, s2);
    s2 = fmaf(v.w, v.w, s2);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) s2 += __shfl_xor(s2, off, 32);
    return sqrtf(s2);
}

// log(1 + x) for x > -1.  Below |x| < 1/16 the Taylor series to x^6 (its
// truncation is under 1e-8 of the result; 1.1e-7 relative in fp32), where
// the hardware log of the rounded 1 + x would lose the small x; above it the
// hardware log (9e-7 relative at worst, near 1/16).  About a tenth of the
// instructions of the full-precision log1pf.
__device__ __forceinline__ float log1p_f32(float x)
{
    if (fabsf(x) < 0.0625f) {
        float r = 1.0f / 6.0f;
        r = 0.2f - x * r;
        r = 0.25f - x * r;
        r = (1.0f / 3.0f) - x * r;
        r = 0.5f - x * r;
        r = 1.0f - x * r;
        return x * r;
    }
    return __logf(1.0f + x);
}

// log u for u = P[at least 2 of L tables collide], P = p^K (fp32).
// Closed form 1 - (1-P)^L - L P (1-P)^(L-1) where L*P > 0.05; below that the
// two subtractions cancel, so u is the binomial tail
//   C(L,2) P^2 (1-P)^(L-2) (1 + c3 r (1 + c4 r (1 + c5 r (1 + c6 r (1 + c7 r))))),
//   r = P/(1-P), c_i = (L-i+1)/i (uc[i-3], from the host; 0 past L),
// taken in logs.  There c_i r <= L P / 3 <= 0.0175 for every i, so the terms
// left out after i = 7 add less than 2e-10 relative: far below fp32.  p is
// floored at 1e-30: p = 0 only for an exactly anti-parallel centered key,
// which cannot collide in exact arithmetic.  Plain logs, exponentials,
// reciprocals and square roots use the hardware instructions (about 1 ulp),
// the cosine's included; log1p(-P) and the log1p of the tail use log1p_f32,
// and the expm1 of the closed form, which carries the cancellation, the
// full-precision routine.
__device__ __forceinline__ float log_u_f32(float p, int K, int L, const float *uc)
{
    if (K == 0) return 0.0f;
    p = fminf(fmaxf(p, 1e-30f), 1.0f);
    const float logP = float(K) * __logf(p);
    const float P = __expf(logP);
    if (P >= 1.0f) return 0.0f;
    const float a = log1p_f32(-P);
    const float LP = float(L) * P;
    if (LP > 0.05f) {
        const float u = -expm1f(float(L) * a) - LP * __expf(float(L - 1) * a);
        return __logf(u);
    }
    const float r = P * __builtin_amdgcn_rcpf(1.0f - P);
    float f = fmaf(uc[4] * r, 1.0f, 1.0f);
    f = fmaf(uc[3] * r, f, 1.0f);
    f = fmaf(uc[2] * r, f, 1.0f);
    f = fmaf(uc[1] * r, f, 1.0f);
    const float rest = uc[0] * r * f;   // the tail after the j = 2 term, relative to it
    return __logf(0.5f * float(L) * float(L - 1)) + 2.0f * logP + float(L - 2) * a + log1p_f32(rest);
}

// arccos(x) / pi for x in [-1, 1], from the minimax form of Abramowitz and
// Stegun 4.4.46: on [0, 1], arccos(x) = sqrt(1 - x) (a0 + a1 x + ... + a7 x^7)
// with absolute error at most 2e-8; arccos(-x) = pi - arccos(x).
__device__ __forceinline__ float acos_over_pi(float x)
{
    const float ax = fabsf(x);
    float r = -0.0012624911f;
    r = fmaf(r, ax, 0.0066700901f);
    r = fmaf(r, ax, -0.0170881256f);
    r = fmaf(r, ax, 0.0308918810f);
    r = fmaf(r, ax, -0.0501743046f);
    r = fmaf(r, ax, 0.0889789874f);
    r = fmaf(r, ax, -0.2145988016f);
    r = fmaf(r, ax, 1.5707963050f);
    r *= __builtin_amdgcn_sqrtf(1.0f - ax);
    const float inv_pi = 0.31830988618379067f;
    return x >= 0.0f ? r * inv_pi : 1.0f - r * inv_pi;
}

// Full-rate cross-lane move inside a DPP row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes; every lane of the group gets it.
// Butterfly over lane ^ 1, lane ^ 2 (quad permutes), then the half-row and
// row mirrors, which pair the two quads of each half and the two halves.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror
    return v;
}

// Max / sum over the wave (64 lanes), the same value in every lane: DPP
// inside each row of 16 lanes, then the four row results in lane order.
__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                       __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ float wave_sum(float v)
{
    v = row16_sum(v);
    const int b = __float_as_int(v);
    return ((__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
             __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
            __int_as_float(__builtin_amdgcn_readlane(b, 32))) +
           __int_as_float(__builtin_amdgcn_readlane(b, 48));
}


// q_g.mu of the G staged queries into sqn[G + g], for q_g.(k - mu) =
// q_g.k - q_g.mu: wave w of the 256 threads takes heads w, w + 4, ..., each
// lane two dims, then a sum over the wave.
template <int G>
__device__ __forceinline__ void stage_qmu(const float (*sq)[kD], const float *smu, float *sqn,
                                          int t)
{
    const int lane = t & 63;
    for (int g = uniform(t >> 6); g < G; g += 4) {
        const float2 qv = reinterpret_cast<const float2 *>(sq[g])[lane];
        const float2 mv = reinterpret_cast<const float2 *>(smu)[lane];
        const float qm = wave_sum(fmaf(qv.x, mv.x, qv.y * mv.y));
        if (lane == 0) sqn[G + g] = qm;
    }
}

// LDS of one gather round: per listed row the three reduced products, per
// (row, head) z and the weight exp(z - running max), and the row's V.
template <int G, typename T> struct GatherLds {
    float srow[kRound][G + 1];       // q.k per head, |k-mu|^2
    float sz[kRound][G];             // z, or -inf where the row is not in the head's set
    float sw[kRound][G];             // exp(z - running max), or 0
    __align__(16) T sv[kRound][kD];  // the round's V rows
};

// Thread = (head, pair of dims) slots of one workgroup of 256: its
// accumulator pair and the head's running max and sum (the same in every
// lane of a wave, since a wave owns whole heads).
template <int G> struct GatherAcc {
    static constexpr int kPairs = (G * (kD / 2) + 255) / 256;
    float acc0[kPairs], acc1[kPairs], m[kPairs], l[kPairs];
    __device__ __forceinline__ void reset()
    {
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            acc0[p] = acc1[p] = 0.0f;
            m[p] = -INFINITY;
            l[p] = 0.0f;
        }
    }
};

// K/V row pointers of unit bkv at this lane's 8 dims.
template <typename T>
__device__ __forceinline__ void row_bases(const DecodeArgs &a, int bkv, int li, const T *&kb,
                                          const T *&vb)
{
    const int b = bkv / a.H_kv, h = bkv % a.H_kv;
    kb = static_cast<const T *>(a.k.data) + b * a.k.sb + h * a.k.sh + 8 * li;
    vb = static_cast<const T *>(a.v.data) + b * a.v.sb + h * a.v.sh + 8 * li;
}

// The K/V words of list entries base + gi + 16 r (r < kRowsPerGroup) of a
// chunk.  Past the list every group re-reads the chunk's first key, which is
// never used: the loads stay unconditional.
template <typename T>
__device__ __forceinline__ void load_rows(const DecodeArgs &a, const T *kb, const T *vb,
                                          const uint32_t *ulist, int base, int ne, int chunk,
                                          int gi, typename Row8<T>::raw (&kr)[kRowsPerGroup],
                                          typename Row8<T>::raw (&vr)[kRowsPerGroup])
{
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
        const int e = gi + 16 * r;
        const int64_t i = int64_t(chunk) * kChunk + (e < ne ? (ulist[base + e] & 0xFFFFu) : 0u);
        kr[r] = Row8<T>::load_raw(kb + i * a.k.sn);
        vr[r] = Row8<T>::load_raw(vb + i * a.v.sn);
    }
}

// Marks a round's row registers as read on every path.  A load whose
// register is never read (rows past the list) stays pending in the
// compiler's count, and later code that reuses the register must first wait
// for it, which with in-order counting means waiting for every younger load
// too: the plane batches issued ahead of the next chunk.
template <typename T>
__device__ __forceinline__ void retire_rows(const typename Row8<T>::raw (&kr)[kRowsPerGroup],
                                            const typename Row8<T>::raw (&vr)[kRowsPerGroup])
{
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
#pragma unroll
        for (int j = 0; j < Row8<T>::kLoads; ++j) asm volatile("" ::"v"(kr[r].w[j]), "v"(vr[r].w[j]));
}

// One round over list entries [base, base + ne), ne <= kRound, whose K/V
// words are kr / vr.  sq: the G queries; sqn: their norms |q_g|, then q_g.mu,
// then the unit's lift radius r (an index built with the lift); smu: mu.
// Three steps:
//   c1: 16 groups of 16 lanes, lane = 8 dims; group gi takes rows gi, gi+16,
//       ... of the round, stages its V rows in LDS and reduces q_g.k and
//       |k - mu|^2 over its lanes (q_g.(k - mu) is q_g.k - q_g.mu);
//   z:  the group's lanes share out its (row, head) pairs and evaluate z for
//       each: on T, z = q.k*scale; on S, z = q.k*scale - log u with
//       p = 1 - acos(cos(q, k - mu))/pi;
//   (barrier)
//   c2: wave w owns heads w, w+4, ...: it forms the round's max, the weights
//       exp(z - max) and their sum, and each thread = (head, pair of dims)
//       rescales its accumulator and adds the weighted V rows;
//   (barrier: the round's LDS may then be rewritten).
// c1 and z of a group touch only LDS that the group's own wave writes, so
// they need no barrier between them.

// c1 for the group's rows gi + 16 r, r in [r0, r1).
template <int G, typename T>
__device__ __forceinline__ void gather_c1(GatherLds<G, T> &s, int ne, const float (*sq)[kD],
                                          const float *smu,
                                          const typename Row8<T>::raw (&kr_)[kRowsPerGroup],
                                          const typename Row8<T>::raw (&vr_)[kRowsPerGroup],
                                          int gi, int li, int r0, int r1)
{
    const float4 m0 = reinterpret_cast<const float4 *>(smu)[2 * li];
    const float4 m1 = reinterpret_cast<const float4 *>(smu)[2 * li + 1];
    const float mu8[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r) {
        const int e = gi + 16 * r;
        if (r < r0 || r >= r1 || e >= ne) continue;   // uniform over the 16-lane group
        Row8<T>::store_raw(&s.sv[e][8 * li], vr_[r]);
        float kr[8];
        Row8<T>::convert(kr_[r], kr);
        float xx = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = kr[j] - mu8[j];
            xx = fmaf(x, x, xx);
        }
        float sd[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float4 q0 = *reinterpret_cast<const float4 *>(&sq[g][8 * li]);
            const float4 q1 = *reinterpret_cast<const float4 *>(&sq[g][8 * li + 4]);
            const float qg[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float s0 = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s0 = fmaf(qg[j], kr[j], s0);
            sd[g] = row16_sum(s0);
        }
        xx = row16_sum(xx);
        if (li == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) s.srow[e][g] = sd[g];
            s.srow[e][G] = xx;
        }
    }
}

// z of the group's (row, head) pairs, one per lane (srow was written by this
// wave: LDS keeps a wave's accesses in order).
template <int G, typename T>
__device__ __forceinline__ void gather_z(const DecodeArgs &a, GatherLds<G, T> &s,
                                         const uint32_t *ulist, int base, int ne,
                                         const float *sqn, int gi, int li)
{
    constexpr int kZ = kRowsPerGroup * G;   // (row, head)s per group
#pragma unroll
    for (int k = 0; k < (kZ + 15) / 16; ++k) {
        const int zp = li + 16 * k;
        const int r = zp / G, g = zp % G;
        const int e = gi + 16 * r;
        if (zp < kZ && e < ne) {
            const uint32_t ent = ulist[base + e];
            const bool exact = (ent >> 24) & 1u;
            float z = -INFINITY;
            if (exact || ((ent >> (16 + g)) & 1u)) {
                z = s.srow[e][g] * a.scale;
                if (!exact) {
                    // q.(k - mu) = q.k - q.mu; a lifted key has norm r
                    const float den = sqn[g] * (a.rnorm ? sqn[2 * G] : __builtin_amdgcn_sqrtf(s.srow[e][G]));
                    float cs = den > 0.0f ? (s.srow[e][g] - sqn[G + g]) * __builtin_amdgcn_rcpf(den)
                                          : 0.0f;
                    cs = fminf(fmaxf(cs, -1.0f), 1.0f);
                    const float pc = 1.0f - acos_over_pi(cs);
                    z -= log_u_f32(pc, a.K, a.L, a.ucoef);
                }
            }
            s.sz[e][g] = z;
        }
    }
}

// c2 (after a barrier that makes every group's z visible).
template <int G, typename T>
__device__ __forceinline__ void gather_c2(GatherLds<G, T> &s, int ne, GatherAcc<G> &acc, int t)
{
    const int lane = t & 63;
#pragma unroll
    for (int p = 0; p < GatherAcc<G>::kPairs; ++p) {
        const int g = uniform((t + 256 * p) / (kD / 2)), dp = lane;
        if (g < G) {
            const float z = lane < ne ? s.sz[lane][g] : -INFINITY;
            const float m_new = fmaxf(acc.m[p], wave_max(z));
            const float wgt = z == -INFINITY ? 0.0f : __expf(z - m_new);
            if (lane < ne) s.sw[lane][g] = wgt;
            const float sc = m_new == -INFINITY ? 1.0f : __expf(acc.m[p] - m_new);
            acc.l[p] = fmaf(acc.l[p], sc, wave_sum(wgt));
            acc.m[p] = m_new;
            // the weights were written by this wave: in order in LDS
            float x0 = acc.acc0[p] * sc, x1 = acc.acc1[p] * sc;
            for (int e = 0; e < ne; ++e) {
                const float wg = s.sw[e][g];
                float v0, v1;
                Row8<T>::load_pair(&s.sv[e][2 * dp], v0, v1);
                x0 = fmaf(wg, v0, x0);
                x1 = fmaf(wg, v1, x1);
            }
            acc.acc0[p] = x0;
            acc.acc1[p] = x1;
        }
    }
}

// kLate: a round after the first, whose rows may be the youngest loads: all
// of them are marked read before c1 (where they are live in any case), rows
// past the list included.
template <int G, typename T, bool kLate>
__device__ __forceinline__ void gather_round(const DecodeArgs &a, GatherLds<G, T> &s,
                                             const uint32_t *ulist, int base, int ne,
                                             const float (*sq)[kD], const float *sqn,
                                             const float *smu,
                                             const typename Row8<T>::raw (&kr_)[kRowsPerGroup],
                                             const typename Row8<T>::raw (&vr_)[kRowsPerGroup],
                                             GatherAcc<G> &acc, int t, int gi, int li)
{
    if (kLate) retire_rows<T>(kr_, vr_);
    gather_c1<G, T>(s, ne, sq, smu, kr_, vr_, gi, li, 0, kRowsPerGroup);
    gather_z<G, T>(a, s, ulist, base, ne, sqn, gi, li);
    __syncthreads();
    gather_c2<G, T>(s, ne, acc, t);
    __syncthreads();   // srow, sz, sw, sv are rewritten by the next round
}

// A chunk's gather in two parts, for a caller that runs the first inside
// other work.  gather_head: round 0's c1 and z, which touch only LDS of the
// calling wave and need no barrier; then, after a barrier, gather_tail: round
// 0's c2 and the later rounds, folded into the caller's accumulator.
template <int G, typename T>
__device__ __forceinline__ void gather_head(const DecodeArgs &a, GatherLds<G, T> &s,
                                            const uint32_t *ulist, int total,
                                            const float (*sq)[kD], const float *sqn,
                                            const float *smu,
                                            const typename Row8<T>::raw (&kr0)[kRowsPerGroup],
                                            const typename Row8<T>::raw (&vr0)[kRowsPerGroup],
                                            int gi, int li)
{
    if (total <= 0) return;
    const int ne = min(kRound, total);
    gather_c1<G, T>(s, ne, sq, smu, kr0, vr0, gi, li, 0, kRowsPerGroup);
    gather_z<G, T>(a, s, ulist, 0, ne, sqn, gi, li);
}

template <int G, bool kCoherent = false>
__device__ __forceinline__ void gather_store(const DecodeArgs &a, const GatherAcc<G> &acc,
                                             int slot, int bkv, int t);

template <int G, typename T>
__device__ __forceinline__ void gather_tail(const DecodeArgs &a, GatherLds<G, T> &s,
                                            const uint32_t *ulist, int total, int chunk, int bkv,
                                            const float (*sq)[kD], const float *sqn,
                                            const float *smu, GatherAcc<G> &acc, int t, int gi,
                                            int li)
{
    if (total > 0) gather_c2<G, T>(s, min(kRound, total), acc, t);
    if (total > kRound) {
        __syncthreads();   // round 0's c2 may still read its LDS
        const T *kb, *vb;
        row_bases<T>(a, bkv, li, kb, vb);
        typename Row8<T>::raw kr[kRowsPerGroup], vr[kRowsPerGroup];
        for (int base = kRound; base < total; base += kRound) {
            const int ne = min(kRound, total - base);
            load_rows<T>(a, kb, vb, ulist, base, ne, chunk, gi, kr, vr);
            gather_round<G, T, true>(a, s, ulist, base, ne, sq, sqn, smu, kr, vr, acc, t, gi, li);
        }
    }
}

// Two floats as one 64-bit word, low word first (their order in memory).
__device__ __forceinline__ uint64_t pack2(float lo, float hi)
{
    return uint64_t(__float_as_uint(lo)) | (uint64_t(__float_as_uint(hi)) << 32);
}

// A partial softmax (max, sum, unnormalised accumulator) per head, into
// record `slot` of unit bkv (records are n_chunks apart per unit; a record
// holds one chunk, or several chunks of one unit folded together).
// kCoherent: stored with device-scope atomic stores (written through to the
// level every XCD reads), for a workgroup that reads the record back within
// the same kernel; every pair of floats is 8-byte aligned (records and
// heads are whole multiples of 8 bytes apart).
template <int G, bool kCoherent>
__device__ __forceinline__ void gather_store(const DecodeArgs &a, const GatherAcc<G> &acc,
                                             int slot, int bkv, int t)
{
    const int lane = t & 63;
    float *part0 = a.part + (int64_t(bkv) * a.n_chunks + slot) * (G * kPart);
#pragma unroll
    for (int p = 0; p < GatherAcc<G>::kPairs; ++p) {
        const int g = uniform((t + 256 * p) / (kD / 2)), dp = lane;
        if (g < G) {
            if constexpr (kCoherent) {
                __hip_atomic_store(reinterpret_cast<uint64_t *>(part0 + g * kPart + 2 + 2 * dp),
                                   pack2(acc.acc0[p], acc.acc1[p]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (dp == 0)
                    __hip_atomic_store(reinterpret_cast<uint64_t *>(part0 + g * kPart),
                                       pack2(acc.m[p], acc.l[p]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            } else {
                part0[g * kPart + 2 + 2 * dp] = acc.acc0[p];
                part0[g * kPart + 3 + 2 * dp] = acc.acc1[p];
                if (dp == 0) {
                    part0[g * kPart] = acc.m[p];
                    part0[g * kPart + 1] = acc.l[p];
                }
            }
        }
    }
}

// The whole list of one chunk, folded into acc: round 0 from rows already
// loaded (kr0 / vr0), later rounds load theirs.  kAhead: the second round's
// rows are issued before the first round runs, so that their latency
// overlaps it (for callers with the registers to spare).
template <int G, typename T, bool kAhead>
__device__ __forceinline__ void gather_chunk_into(const DecodeArgs &a, GatherLds<G, T> &s,
                                                  const uint32_t *ulist, int total, int chunk,
                                                  int bkv, const float (*sq)[kD],
                                                  const float *sqn, const float *smu,
                                                  const typename Row8<T>::raw (&kr0)[kRowsPerGroup],
                                                  const typename Row8<T>::raw (&vr0)[kRowsPerGroup],
                                                  GatherAcc<G> &acc, int t, int gi, int li)
{
    const T *kb, *vb;
    row_bases<T>(a, bkv, li, kb, vb);
    typename Row8<T>::raw kr[kRowsPerGroup], vr[kRowsPerGroup];
    if (kAhead && total > kRound)
        load_rows<T>(a, kb, vb, ulist, kRound, min(kRound, total - kRound), chunk, gi, kr, vr);
    if (total > 0)
        gather_round<G, T, false>(a, s, ulist, 0, min(kRound, total), sq, sqn, smu, kr0, vr0, acc,
                                  t, gi, li);
    if (total > kRound) {
        __syncthreads();   // the first round's c2 may still read its LDS
        for (int base = kRound; base < total; base += kRound) {
            const int ne = min(kRound, total - base);
            if (!kAhead || base > kRound) load_rows<T>(a, kb, vb, ulist, base, ne, chunk, gi, kr, vr);
            gather_round<G, T, true>(a, s, ulist, base, ne, sq, sqn, smu, kr, vr, acc, t, gi, li);
        }
    }
}

// The merge of one unit's records inside the gather kernel (the scan's, or
// the table path's), by the workgroup that stores the unit's last record
// (runs aligned with units, at most kFusedMergeWide records, G <= 4).  Each
// record was stored with device-scope stores and counted after they
// completed (s_waitcnt), so device-scope loads here find every record,
// whichever XCD wrote it.  Wave w takes head g = w: lane r loads the (max,
// sum) of record r, the wave forms the head's max M, the weights
// w_r = exp(m_r - M) (0 past nrec or for an empty record) and their sum with
// the l_r, and puts the weights in LDS (read back by the same wave: no
// barrier); thread (g, dp) folds the accumulator pairs of every record, all
// NR loads issued before the first is used, in record order.
template <int G, typename T, int NR>
__device__ __forceinline__ void merge_unit_records(const DecodeArgs &a, int bkv, int nrec,
                                                   GatherLds<G, T> &s, int t)
{
    static_assert(G <= 4 && NR <= kRound, "one (head, pair of dims) a thread, a record a lane");
    constexpr int kB = NR < 32 ? NR : 32;   // accumulator loads in flight at once
    const int lane = t & 63, g = t >> 6;
    if (g >= G) return;   // the whole wave
    const float *p0 = a.part + int64_t(bkv) * a.n_chunks * (G * kPart) + g * kPart;
    uint64_t av[kB];
    auto load_batch = [&](int r0) {
#pragma unroll
        for (int r = 0; r < kB; ++r) {
            const int rr = min(r0 + r, nrec - 1);   // past nrec: re-read the last, weight 0
            av[r] = __hip_atomic_load(
                reinterpret_cast<const uint64_t *>(p0 + int64_t(rr) * (G * kPart) + 2 + 2 * lane),
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    load_batch(0);
    const uint64_t ml = __hip_atomic_load(
        reinterpret_cast<const uint64_t *>(p0 + int64_t(min(lane, nrec - 1)) * (G * kPart)),
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float m = lane < nrec ? __uint_as_float(uint32_t(ml)) : -INFINITY;
    const float l = lane < nrec ? __uint_as_float(uint32_t(ml >> 32)) : 0.0f;
    const float M = wave_max(m);
    const float wr = m == -INFINITY ? 0.0f : __expf(m - M);
    const float Ls = wave_sum(wr * l);
    if (lane < NR) s.sw[lane][g] = wr;
    float x0 = 0.0f, x1 = 0.0f;
#pragma unroll 1
    for (int r0 = 0; r0 < NR; r0 += kB) {   // one batch of loads live at a time
        if (r0 > 0) load_batch(r0);
#pragma unroll
        for (int r = 0; r < kB; ++r) {
            const float wg = s.sw[r0 + r][g];
            x0 = fmaf(wg, __uint_as_float(uint32_t(av[r])), x0);
            x1 = fmaf(wg, __uint_as_float(uint32_t(av[r] >> 32)), x1);
        }
    }
    const int b = bkv / a.H_kv, h = bkv % a.H_kv;
    reinterpret_cast<float2 *>(a.out + (int64_t(b) * a.H_q + h * G + g) * kD)[lane] =
        Ls > 0.0f ? make_float2(x0 / Ls, x1 / Ls) : make_float2(0.0f, 0.0f);
}

// Records a unit has when its runs (cpb chunks; 1 on the table path) align
// with it, for the fused merge, or 0 where the separate merge kernel runs
// instead.  The fused merge reads a unit's records on one workgroup after
// that unit's last run.  It takes up to 32 records a unit; at 32 (16K
// context) the step is 0.7-0.9 us shorter than with the merge kernel, at 4
// (batch 16 x 32K) 1-3%.  With 64 records and few units (96K: 8) the last
// workgroups' reads of 131 KB each made scan_gather 3.3 us longer and the
// step 0.3-0.9 us longer; with 64 and many units (the table path at batch 16:
// 128) the merges spread over as many CUs and replace a merge kernel of 4,096
// blocks, so up to 64 are taken there.
// The code scan takes at most kFusedMergeMax (its runs give more than that
// only with few units), the table path up to kFusedMergeWide.
constexpr int kFusedMergeMax = 32, kFusedMergeWide = 64, kFusedWideUnits = 32;
inline int fused_merge_records(const DecodeArgs &a, int G, int cpb, int max_rec)
{
    if (G > 4 || !a.unit_cnt || a.n_chunks % cpb != 0) return 0;
    const int nrec = a.n_chunks / cpb;
    if (nrec <= kFusedMergeMax) return nrec;
    return nrec <= max_rec && a.B * a.H_kv >= kFusedWideUnits ? nrec : 0;
}

// A workgroup's record of unit bkv (record rec of nrec), stored so that the
// workgroup that stores the unit's last record can merge them all in this
// kernel: device-scope stores, a wait for their completion, then the unit's
// count (a device-scope add; the counts start at zero).  Every thread calls
// it; flag is an LDS word.
template <int G, typename T, int kMaxRec>
__device__ __forceinline__ void store_count_merge(const DecodeArgs &a, const GatherAcc<G> &acc,
                                                  int rec, int bkv, int nrec, GatherLds<G, T> &s,
                                                  int *flag, int t)
{
    static_assert(kMaxRec == kFusedMergeMax || kMaxRec == kFusedMergeWide, "a merge width");
    if constexpr (G <= 4) {
        gather_store<G, true>(a, acc, rec, bkv, t);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t == 0)
            *flag = __hip_atomic_fetch_add(a.unit_cnt + bkv, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == nrec - 1;
        __syncthreads();
        if (*flag) {
            if (nrec <= 8) merge_unit_records<G, T, 8>(a, bkv, nrec, s, t);
            else if (nrec <= 16) merge_unit_records<G, T, 16>(a, bkv, nrec, s, t);
            else if (kMaxRec == kFusedMergeMax || nrec <= kFusedMergeMax)
                merge_unit_records<G, T, kFusedMergeMax>(a, bkv, nrec, s, t);
            else merge_unit_records<G, T, kMaxRec>(a, bkv, nrec, s, t);
        }
    }
}

// Ascending compaction of a chunk's flagged keys: thread t owns keys 2t and
// 2t+1 and hands in their flags and list entries (key | headmask << 16 |
// exact << 24).  Writes ulist and returns the list length (every thread).
__device__ __forceinline__ int compact_list(bool fl0, bool fl1, uint32_t ent0, uint32_t ent1,
                                            uint32_t *ulist, int *wsum, int t)
{
    const int lane = t & 63, w = t >> 6;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const unsigned long long b0 = __ballot(fl0), b1 = __ballot(fl1);
    const int pre = __popcll(b0 & lt) + __popcll(b1 & lt);
    if (lane == 0) wsum[w] = __popcll(b0) + __popcll(b1);
    __syncthreads();
    int woff = 0;
    for (int j = 0; j < w; ++j) woff += wsum[j];
    const int pos = woff + pre;
    if (fl0) ulist[pos] = ent0;
    if (fl1) ulist[pos + (fl0 ? 1 : 0)] = ent1;
    return wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// Debug view: per-head sampled keys of a chunk (ascending) into seg_idx /
// seg_cnt; hm0 / hm1 are the head masks of keys key0, key0 + 1.
template <int G>
__device__ __forceinline__ void write_seg_lists(const DecodeArgs &a, uint32_t hm0, uint32_t hm1,
                                                int64_t key0, int bhq0, int chunk, int *wsum,
                                                int t)
{
    const int lane = t & 63, w = t >> 6;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g = 0; g < G; ++g) {
        const bool s0 = (hm0 >> g) & 1u, s1 = (hm1 >> g) & 1u;
        const unsigned long long b0 = __ballot(s0), b1 = __ballot(s1);
        const int pre = __popcll(b0 & lt) + __popcll(b1 & lt);
        __syncthreads();
        if (lane == 0) wsum[w] = __popcll(b0) + __popcll(b1);
        __syncthreads();
        int woff = 0;
        for (int j = 0; j < w; ++j) woff += wsum[j];
        int32_t *seg = a.seg_idx + (int64_t(bhq0 + g) * a.n_chunks + chunk) * kChunk;
        if (s0) seg[woff + pre] = int32_t(key0);
        if (s1) seg[woff + pre + (s0 ? 1 : 0)] = int32_t(key0 + 1);
        if (t == 0)
            a.seg_cnt[int64_t(bhq0 + g) * a.n_chunks + chunk] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    }
}

}  // namespace
}  // namespace mp
