// decode.hip -- one MagicPIG decode step on gfx950: three launches.
//
//   encode_query   SimHash codes of the raw queries (page "MagicPIG: LSH
//                  Sampling for Efficient LLM Generation", algorithm steps:
//                  the query's code from the shared projector).
//   scan_gather    a workgroup takes a run of 512-key chunks (each of one KV
//                  head and its G query heads), as many workgroups as are
//                  resident at once; per chunk:
//                  (a) stream the chunk's codes (16-byte lane loads) and count,
//                      per key and query head, the tables where the key shares
//                      the query's bucket;
//                  (b) a key is sampled for a head iff that count is >= 2 and
//                      the key is not in the exact set T (method details and
//                      page "MagicPIG: don't pick the tallest", section 5);
//                      ballot/prefix-sum compaction of the union of sampled
//                      and exact keys into an ascending LDS list;
//                  (c) gather the listed K/V rows, recompute q.k and the cosine
//                      to the centered key, u_i = P[Binomial(L, p^K) >= 2],
//                      z = q.k*scale - log u (z = q.k*scale on T), and run an
//                      online softmax per query head (algorithm steps: one
//                      softmax over [w_S, w_T]/sqrt(d) - log[u, 1]); the
//                      chunk's partial softmax (max, sum, unnormalised
//                      accumulator) per head goes to scratch.
//                  The code stream runs two batches ahead across chunks, and
//                  (c) runs one chunk late, so a chunk's rows arrive while the
//                  next chunk is scanned.
//   merge          log-sum-exp merge of the chunk partials of every query head
//                  (system co-design: partial attention outputs are merged
//                  recursively).  A kernel of its own: its launch boundary is
//                  what makes the partials of blocks on other XCDs visible,
//                  which an in-kernel device-scope fence would buy with an L2
//                  write-back per block.
#include <hip/hip_ext.h>
#include <math.h>

#include "mp_internal.h"

namespace mp {
namespace {

constexpr int kPart = kD + 2;     // partial softmax: m, l, acc[128]
#ifndef MP_ROWS_PER_GROUP
#define MP_ROWS_PER_GROUP 4
#endif
constexpr int kRowsPerGroup = MP_ROWS_PER_GROUP;  // listed rows a 16-lane group holds per round
constexpr int kRound = 16 * kRowsPerGroup;
#ifndef MP_SCAN_BATCH
#define MP_SCAN_BATCH 4
#endif
constexpr int kScanBatch = MP_SCAN_BATCH;   // tables per code batch in the scan

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

// Per 16-bit half: min(a, b).  Written out because the compiler turns the
// vector-extension form into compares and selects.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// log u for u = P[at least 2 of L tables collide], P = p^K (fp32).
// Closed form 1 - (1-P)^L - L P (1-P)^(L-1) where L*P > 0.05; below that the
// two subtractions cancel, so u is the binomial tail
//   C(L,2) P^2 (1-P)^(L-2) * (1 + sum_{j>=3} prod_{i=2}^{j-1} (L-i)/(i+1) P/(1-P))
// taken in logs.  p is floored at 1e-30: p = 0 only for an exactly
// anti-parallel centered key, which cannot collide in exact arithmetic.
__device__ __forceinline__ float log_u_f32(float p, int K, int L)
{
    if (K == 0) return 0.0f;
    p = fminf(fmaxf(p, 1e-30f), 1.0f);
    const float logP = float(K) * logf(p);
    const float P = expf(logP);
    if (P >= 1.0f) return 0.0f;
    const float a = log1pf(-P);
    const float LP = float(L) * P;
    if (LP > 0.05f) {
        const float u = -expm1f(float(L) * a) - LP * expf(float(L - 1) * a);
        return logf(u);
    }
    const float r = P / (1.0f - P);
    float term = 1.0f, rest = 0.0f;
    for (int j = 2; j < L; ++j) {
        term *= float(L - j) / float(j + 1) * r;
        rest += term;
        if (term < 1e-9f * (1.0f + rest)) break;
    }
    return logf(0.5f * float(L) * float(L - 1)) + 2.0f * logP + float(L - 2) * a + log1pf(rest);
}

// ---------------------------------------------------------------- query codes
// Block: TB = 64/K whole tables (<= 64 hyperplanes) x 4 query heads.  Lane =
// hyperplane, wave = query head: the lane keeps its W row in registers and
// reads the head's query from LDS (a broadcast).  Sign bits meet in LDS and
// are packed per (head, table).
__global__ __launch_bounds__(256) void encode_query_kernel(const float *__restrict__ q,
                                                           int32_t BHq,
                                                           const float *__restrict__ W, int32_t K,
                                                           int32_t L,
                                                           uint16_t *__restrict__ qcodes,
                                                           uint32_t *__restrict__ qq,
                                                           float *__restrict__ qnorm)
{
    __shared__ float4 sQ[4][kD / 4];
    __shared__ uint8_t sbit[4][64];
    const int t = threadIdx.x;
    const int TB = K > 0 ? 64 / K : 64;
    const int l0 = blockIdx.x * TB;
    const int nt = min(TB, L - l0);
    const int nh = nt * K;
    const int q0 = blockIdx.y * 4;
    const int nq = min(4, BHq - q0);
    const float4 *q4 = reinterpret_cast<const float4 *>(q + int64_t(q0) * kD);
    if (t < nq * (kD / 4)) sQ[t / (kD / 4)][t % (kD / 4)] = q4[t];
    const int hp = t & 63, qi = uniform(t >> 6);
    float4 wr[kD / 4];
    if (hp < nh) {
        const float4 *w4 = reinterpret_cast<const float4 *>(W + (int64_t(l0) * K + hp) * kD);
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) wr[c] = w4[c];
    }
    __syncthreads();
    if (blockIdx.x == 0 && qi < nq) {       // |q| of this wave's head, for the cosines
        const float4 v = sQ[qi][hp & 31];
        float s2 = hp < 32 ? v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w : 0.0f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) s2 += __shfl_xor(s2, off);
        if (hp == 0) qnorm[q0 + qi] = sqrtf(s2);
    }
    if (hp < nh && qi < nq) {
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;   // four chains, dims c mod 4
#pragma unroll
        for (int c = 0; c < kD / 4; ++c) {
            const float4 qv = sQ[qi][c];
            a0 = fmaf(wr[c].x, qv.x, a0);
            a1 = fmaf(wr[c].y, qv.y, a1);
            a2 = fmaf(wr[c].z, qv.z, a2);
            a3 = fmaf(wr[c].w, qv.w, a3);
        }
        sbit[qi][hp] = ((a0 + a1) + (a2 + a3)) > 0.0f ? 1 : 0;
    }
    __syncthreads();
    if (t < nq * nt) {
        const int qj = t / nt, tl = t % nt;
        uint32_t code = 0;
        for (int bb = 0; bb < K; ++bb) code |= uint32_t(sbit[qj][tl * K + bb]) << bb;
        const int64_t o = int64_t(q0 + qj) * L + l0 + tl;
        qcodes[o] = uint16_t(code);
        qq[o] = code | (code << 16);
    }
}

// ---------------------------------------------------------------- scan + gather
// Waves per SIMD the register budget is cut for: 3 up to G = 4 with bf16 rows
// (the next chunk's first code batches stay in registers through a gather),
// 2 otherwise.
#ifndef MP_SCAN_OCC
#define MP_SCAN_OCC 3
#endif
template <int G, typename T>
constexpr int scan_occupancy() { return G <= 2 || (G == 4 && sizeof(T) == 2) ? MP_SCAN_OCC : 2; }

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

// One workgroup takes a run of `cpb` consecutive 512-key chunks (numbered
// over (sequence, KV head) units, then chunks); runs are as equal as the
// chunk count allows and the grid is no larger than what is resident at
// once.  Per chunk:
//   (a) scan: wave w counts the chunk's tables [w L/4, (w+1) L/4);
//   (b) the union of sampled and exact keys is compacted into an ascending
//       LDS list, and the K/V rows of its first kRound entries are loaded;
//   (c) gather-SNIS over the list, run one chunk late: after the next
//       chunk's scan, when the rows have long arrived.  The chunk's partial
//       softmax goes to `part`.
// Each wave reads its tables of all chunks of the run as one stream of
// kScanBatch-table batches in two alternating register buffers, issued two
// batches ahead across chunk boundaries.  Every load on the main path is
// unconditional (padding batches and rows re-read an address already read
// and count nothing), so the compiler can wait on each buffer alone rather
// than on every load in flight.
template <int G, typename T>
__global__ __launch_bounds__(256, (scan_occupancy<G, T>())) void scan_gather_kernel(DecodeArgs a,
                                                                                    int32_t cpb)
{
    __shared__ uint32_t red[G][256];         // packed mismatch counts, word = 2 keys
    __shared__ __align__(16) uint32_t sqq[256][G];   // query codes, code | code << 16
    __shared__ uint32_t ulist[kChunk];       // key | headmask << 16 | exact << 24
    __shared__ int wsum[4];
    __shared__ __align__(16) float sq[2][G][kD];   // per staged unit: the group's queries
    __shared__ float sqn[2][G];              // their norms
    __shared__ __align__(16) float smu[2][kD];   // mean of the unit's keys
    __shared__ float srow[kRound][2 * G + 1];   // per listed row: q.k, q.(k-mu), |k-mu|^2
    __shared__ float sz[kRound][G];          // per (row, head): z, or -inf if not sampled
    __shared__ float sw[kRound][G];          // per (row, head): exp(z - running max) or 0
    __shared__ __align__(16) T sv[kRound][kD];  // the round's V rows

    const int w = uniform(threadIdx.x >> 6);
    const int L = a.L;
    const int gc_begin = blockIdx.x * cpb;
    const int nrun = min(cpb, a.B * a.H_kv * a.n_chunks - gc_begin);
    const int lb = uniform((w * L) / 4), le = uniform(((w + 1) * L) / 4);
    const int lmax = max(le - 1, 0);
    // batches per chunk for this wave: even, and at least 2 (a wave without
    // tables still streams, and counts nothing)
    const int nb = uniform(max(2, ((le - lb + kScanBatch - 1) / kScanBatch + 1) & ~1));
    const uint32_t one2 = 0x00010001u;

    // ---- the code stream: next batch to load is batch ls of chunk lc of the run ----
    u32x4 bufA[kScanBatch], bufB[kScanBatch];
    const int slane = threadIdx.x & 63;
    int lc = 0, ls = 0;
    auto load_next = [&](u32x4(&buf)[kScanBatch]) {
        const bool past = lc >= nrun;                     // beyond the run: re-read the last batch
        const int c = past ? nrun - 1 : lc, sb = past ? nb - 1 : ls;
        const u32x4 *cp = reinterpret_cast<const u32x4 *>(
                               a.codes + int64_t(gc_begin + c) * L * kChunk) + slane;
        const int l0 = lb + sb * kScanBatch;
#pragma unroll
        for (int u = 0; u < kScanBatch; ++u)
            buf[u] = cp[int64_t(min(l0 + u, lmax)) * (kChunk / 8)];
        if (++ls == nb) {
            ls = 0;
            ++lc;
        }
    };
    load_next(bufA);
    load_next(bufB);
    // Wait for both here (nothing else is in flight yet), so that at the top
    // of the chunk loop only the steady-state order of loads is possible:
    // bufA, bufB, then the previous chunk's rows.
    asm volatile("" ::"v"(bufA[0]), "v"(bufA[1]), "v"(bufA[2]), "v"(bufA[3]), "v"(bufB[0]),
                 "v"(bufB[1]), "v"(bufB[2]), "v"(bufB[3]));

    // the chunk whose gather is pending, and its rows
    bool pend = false;
    int p_bkv = 0, p_chunk = 0, p_total = 0, p_slot = 0;
    typename Row8<T>::raw kraw[kRowsPerGroup], vraw[kRowsPerGroup];
    int cur_unit = -1, slot = 1;

#pragma unroll 1
    for (int it = 0; it <= nrun; ++it) {
        // Per-thread offsets are recomputed each chunk from an opaque copy
        // of the thread index: hoisted out of the loop they would hold
        // registers through it.
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int lane = t & 63, gi = t >> 4, li = t & 15;
        const bool scan = it < nrun;
        const int gc = gc_begin + it;
        const int bkv = scan ? gc / a.n_chunks : 0;
        const int chunk = scan ? gc - bkv * a.n_chunks : 0;
        const int bhq0 = (bkv / a.H_kv) * a.H_q + (bkv % a.H_kv) * G;
        if (scan) {
            if (bkv != cur_unit) {
                // A new (sequence, KV head) unit: its query codes for the scan
                // ([table][head], one broadcast per table) and, in the other
                // slot, the queries, norms and mean for its gathers (the
                // pending chunk still reads the current slot).
                slot ^= 1;
                for (int i = t; i < G * L; i += 256) sqq[i % L][i / L] = a.qq[int64_t(bhq0) * L + i];
                for (int i = t; i < G * kD; i += 256)
                    sq[slot][i / kD][i % kD] = a.q[int64_t(bhq0) * kD + i];
                if (t < G) sqn[slot][t] = a.qnorm[bhq0 + t];
                if (t < kD) smu[slot][t] = a.mu[int64_t(bkv) * kD + t];
                cur_unit = bkv;
            }
            for (int i = t; i < G * 256; i += 256) (&red[0][0])[i] = 0u;
            __syncthreads();

            // ---- (a) collision counts ----
            uint32_t mism[4][G];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int g = 0; g < G; ++g) mism[k][g] = 0u;
            auto count_batch = [&](const u32x4(&buf)[kScanBatch], int l0) {
                const int nv = min(kScanBatch, le - l0);
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u) {
                    // padding (u >= nv) adds min(x, 0) = 0 mismatches
                    const uint32_t lim = u < nv ? one2 : 0u;
                    const int lu = min(l0 + u, lmax);
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const uint32_t qv = sqq[lu][g];
                        mism[0][g] += pk_min_u16(buf[u].x ^ qv, lim);
                        mism[1][g] += pk_min_u16(buf[u].y ^ qv, lim);
                        mism[2][g] += pk_min_u16(buf[u].z ^ qv, lim);
                        mism[3][g] += pk_min_u16(buf[u].w ^ qv, lim);
                    }
                }
            };
            // The first pair is peeled: entering it, the previous chunk's
            // round-0 rows are younger than bufA and bufB and need not be
            // waited for; inside the loop only the other buffer is younger.
            count_batch(bufA, lb);
            load_next(bufA);
            count_batch(bufB, lb + kScanBatch);
            load_next(bufB);
            for (int sb = 2; sb < nb; sb += 2) {
                count_batch(bufA, lb + sb * kScanBatch);
                load_next(bufA);
                count_batch(bufB, lb + (sb + 1) * kScanBatch);
                load_next(bufB);
            }
            // Each half counts at most 255 tables, so a 32-bit add of the
            // packed pair never carries between keys.
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int g = 0; g < G; ++g) atomicAdd(&red[g][lane * 4 + k], mism[k][g]);
        }

        if (!scan && pend) {
            // Past the run the rows are the youngest loads: wait for them on
            // this path alone, so that where the paths meet the rows count
            // as older than the two batches in flight.
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r)
#pragma unroll
                for (int j = 0; j < Row8<T>::kLoads; ++j)
                    asm volatile("" ::"v"(kraw[r].w[j]), "v"(vraw[r].w[j]));
        }
        if (pend) {
            // ---- (c) gather-SNIS of the pending chunk, in rounds of up to
            // kRound listed rows (round 0's rows are already loaded) ----
            // c1: 16 groups of 16 lanes, lane = 8 dims; group gi takes rows
            //     gi, gi+16, ... of the round, stages its V rows in LDS and
            //     reduces q_g.k, q_g.(k - mu) and |k - mu|^2 over its lanes;
            //     the group's lanes then share out its (row, head) pairs and
            //     evaluate z for each;
            // c2: wave w owns heads w, w+4, ... (their running max and sum live
            //     in its registers): it forms the round's max, the weights
            //     exp(z - max) and their sum, and each thread = (head, pair of
            //     dims) rescales its accumulator and adds the weighted V rows.
            const int pb = p_bkv / a.H_kv, ph = p_bkv % a.H_kv;
            const T *kb = static_cast<const T *>(a.k.data) + pb * a.k.sb + ph * a.k.sh + 8 * li;
            const T *vb = static_cast<const T *>(a.v.data) + pb * a.v.sb + ph * a.v.sh + 8 * li;
            constexpr int kPairs = (G * (kD / 2) + 255) / 256;   // (head, dim pair)s per thread
            constexpr int kZ = kRowsPerGroup * G;                 // (row, head)s per group
            float acc0[kPairs], acc1[kPairs], m_run[kPairs], l_run[kPairs];
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                acc0[p] = acc1[p] = 0.0f;
                m_run[p] = -INFINITY;
                l_run[p] = 0.0f;
            }
            const float inv_pi = 0.31830988618379067f;
            using Raw = typename Row8<T>::raw;
            // One round: rows [base, base + ne) of the list, their K/V words in kr_/vr_.
            auto round = [&](int base, const Raw(&kr_)[kRowsPerGroup], const Raw(&vr_)[kRowsPerGroup]) {
                const int ne = min(kRound, p_total - base);
                const float4 m0 = reinterpret_cast<const float4 *>(smu[p_slot])[2 * li];
                const float4 m1 = reinterpret_cast<const float4 *>(smu[p_slot])[2 * li + 1];
                const float mu8[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                for (int r = 0; r < kRowsPerGroup; ++r) {
                    const int e = gi + 16 * r;
                    if (e >= ne) continue;            // uniform over the 16-lane group
                    Row8<T>::store_raw(&sv[e][8 * li], vr_[r]);
                    float kr[8], x[8];
                    Row8<T>::convert(kr_[r], kr);
                    float xx = 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        x[j] = kr[j] - mu8[j];
                        xx = fmaf(x[j], x[j], xx);
                    }
                    float sd[G], td[G];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float4 q0 = *reinterpret_cast<const float4 *>(&sq[p_slot][g][8 * li]);
                        const float4 q1 =
                            *reinterpret_cast<const float4 *>(&sq[p_slot][g][8 * li + 4]);
                        const float qg[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                        float s0 = 0.0f, t0 = 0.0f;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            s0 = fmaf(qg[j], kr[j], s0);
                            t0 = fmaf(qg[j], x[j], t0);
                        }
                        sd[g] = row16_sum(s0);
                        td[g] = row16_sum(t0);
                    }
                    xx = row16_sum(xx);
                    if (li == 0) {
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            srow[e][g] = sd[g];
                            srow[e][G + g] = td[g];
                        }
                        srow[e][2 * G] = xx;
                    }
                }
                // z of the group's (row, head) pairs, one per lane (srow was
                // written by this wave: LDS keeps a wave's accesses in order)
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
                            z = srow[e][g] * a.scale;
                            if (!exact) {
                                const float den = sqn[p_slot][g] * sqrtf(srow[e][2 * G]);
                                float cs = den > 0.0f ? srow[e][G + g] / den : 0.0f;
                                cs = fminf(fmaxf(cs, -1.0f), 1.0f);
                                const float pc = 1.0f - acosf(cs) * inv_pi;
                                z -= log_u_f32(pc, a.K, L);
                            }
                        }
                        sz[e][g] = z;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int p = 0; p < kPairs; ++p) {
                    const int g = uniform((t + 256 * p) / (kD / 2)), dp = lane;
                    if (g < G) {
                        const float z = lane < ne ? sz[lane][g] : -INFINITY;
                        const float m_new = fmaxf(m_run[p], wave_max(z));
                        const float wgt = z == -INFINITY ? 0.0f : __expf(z - m_new);
                        if (lane < ne) sw[lane][g] = wgt;
                        const float sc = m_new == -INFINITY ? 1.0f : __expf(m_run[p] - m_new);
                        l_run[p] = fmaf(l_run[p], sc, wave_sum(wgt));
                        m_run[p] = m_new;
                        // the weights were written by this wave: in order in LDS
                        float x0 = acc0[p] * sc, x1 = acc1[p] * sc;
                        for (int e = 0; e < ne; ++e) {
                            const float wg = sw[e][g];
                            float v0, v1;
                            Row8<T>::load_pair(&sv[e][2 * dp], v0, v1);
                            x0 = fmaf(wg, v0, x0);
                            x1 = fmaf(wg, v1, x1);
                        }
                        acc0[p] = x0;
                        acc1[p] = x1;
                    }
                }
                __syncthreads();   // srow, sz, sw, sv are rewritten by the next round
            };
            // Round 0 with the rows loaded before the scan (older than the
            // batches in flight); later rounds load theirs here.
            if (p_total > 0) round(0, kraw, vraw);
            for (int base = kRound; base < p_total; base += kRound) {
                const int ne = min(kRound, p_total - base);
                Raw kr2[kRowsPerGroup], vr2[kRowsPerGroup];
#pragma unroll
                for (int r = 0; r < kRowsPerGroup; ++r) {
                    const int e = gi + 16 * r;
                    const int64_t i = int64_t(p_chunk) * kChunk +
                                      (e < ne ? (ulist[base + e] & 0xFFFFu) : 0u);
                    kr2[r] = Row8<T>::load_raw(kb + i * a.k.sn);
                    vr2[r] = Row8<T>::load_raw(vb + i * a.v.sn);
                }
                round(base, kr2, vr2);
            }
            // the chunk's partial: (max, sum, unnormalised accumulator) per head
            float *part0 = a.part + (int64_t(p_bkv) * a.n_chunks + p_chunk) * (G * kPart);
#pragma unroll
            for (int p = 0; p < kPairs; ++p) {
                const int g = uniform((t + 256 * p) / (kD / 2)), dp = lane;
                if (g < G) {
                    part0[g * kPart + 2 + 2 * dp] = acc0[p];
                    part0[g * kPart + 3 + 2 * dp] = acc1[p];
                    if (dp == 0) {
                        part0[g * kPart] = m_run[p];
                        part0[g * kPart + 1] = l_run[p];
                    }
                }
            }
        }
        // counts in red are complete; the pending chunk's list is no longer
        // read
        __syncthreads();
        pend = false;
        if (!scan) break;

        // ---- (b) sampled / exact sets and ascending compaction ----
        // Thread t owns keys 2t and 2t+1 of the chunk.
        const int n = a.n;
        const int64_t key0 = int64_t(chunk) * kChunk + 2 * t;
        uint32_t hm[2] = {0u, 0u};
        bool ex[2], fl[2];
        uint32_t cnt[2][G];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t i = key0 + e;
            const bool valid = i < n;
            ex[e] = valid && (i < a.n_sink || i >= int64_t(n) - a.n_local);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint32_t mm = (red[g][t] >> (16 * e)) & 0xFFFFu;
                cnt[e][g] = uint32_t(L) - mm;
                if (valid && !ex[e] && cnt[e][g] >= 2u) hm[e] |= 1u << g;
            }
            fl[e] = ex[e] || hm[e] != 0u;
        }
        const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        {
            const unsigned long long b0 = __ballot(fl[0]), b1 = __ballot(fl[1]);
            const int pre = __popcll(b0 & lt) + __popcll(b1 & lt);
            if (lane == 0) wsum[w] = __popcll(b0) + __popcll(b1);
            __syncthreads();
            int woff = 0;
            for (int j = 0; j < w; ++j) woff += wsum[j];
            const int pos = woff + pre;
            if (fl[0]) ulist[pos] = uint32_t(2 * t) | (hm[0] << 16) | (uint32_t(ex[0]) << 24);
            if (fl[1])
                ulist[pos + (fl[0] ? 1 : 0)] =
                    uint32_t(2 * t + 1) | (hm[1] << 16) | (uint32_t(ex[1]) << 24);
        }
        const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];

        if (a.debug) {
            if (a.counts) {
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (key0 + e < n)
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            a.counts[int64_t(bhq0 + g) * n + key0 + e] = uint8_t(cnt[e][g]);
            }
            // Per-head sampled lists of this chunk (ascending), for the S view.
            for (int g = 0; g < G; ++g) {
                const bool s0 = (hm[0] >> g) & 1u, s1 = (hm[1] >> g) & 1u;
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
                    a.seg_cnt[int64_t(bhq0 + g) * a.n_chunks + chunk] =
                        wsum[0] + wsum[1] + wsum[2] + wsum[3];
            }
        }
        __syncthreads();   // ulist complete

        // Round 0's rows of this chunk, in flight during the next scan.  Every
        // group loads kRowsPerGroup rows; past the list it re-reads the
        // chunk's first key, which is never used.
        {
            const int b = bkv / a.H_kv, h = bkv % a.H_kv;
            const T *kb = static_cast<const T *>(a.k.data) + b * a.k.sb + h * a.k.sh + 8 * li;
            const T *vb = static_cast<const T *>(a.v.data) + b * a.v.sb + h * a.v.sh + 8 * li;
            const int ne = min(kRound, total);
#pragma unroll
            for (int r = 0; r < kRowsPerGroup; ++r) {
                const int e = gi + 16 * r;
                const int64_t i =
                    int64_t(chunk) * kChunk + (e < ne ? (ulist[e] & 0xFFFFu) : 0u);
                kraw[r] = Row8<T>::load_raw(kb + i * a.k.sn);
                vraw[r] = Row8<T>::load_raw(vb + i * a.v.sn);
            }
        }
        pend = true;
        p_bkv = bkv;
        p_chunk = chunk;
        p_total = total;
        p_slot = slot;
    }
}

// ---------------------------------------------------------------- merge
// Block = one (KV head unit, query head g of its group, quarter of the dims);
// thread = (dim c of 32, chunk lane j of 32).  Lane j folds chunks j, j+32,
// ... into a running (max, sum, acc) in one pass; the 32 lanes are then
// combined in lane order, so the result is deterministic.
template <int G>
__global__ __launch_bounds__(1024) void merge_kernel(const float *__restrict__ part,
                                                    int32_t n_chunks, int32_t H_kv, int32_t H_q,
                                                    float *__restrict__ out)
{
    __shared__ float sm[32][33], sl[32][33], sa[32][33];
    const int bkv = blockIdx.x / G, g = blockIdx.x % G;
    const int t = threadIdx.x, cl = t & 31, j = t >> 5;
    const int c = 32 * blockIdx.y + cl;
    const float *p = part + int64_t(bkv) * n_chunks * (G * kPart) + g * kPart;
    float m = -INFINITY, l = 0.0f, acc = 0.0f;
#pragma unroll 2
    for (int ch = j; ch < n_chunks; ch += 32) {
        const float *pc = p + int64_t(ch) * (G * kPart);
        const float mc = pc[0], lc = pc[1], ac = pc[2 + c];
        if (mc > m) {
            const float f = __expf(m - mc);      // 0 while m = -inf
            l = fmaf(l, f, lc);
            acc = fmaf(acc, f, ac);
            m = mc;
        } else if (mc != -INFINITY) {
            const float f = __expf(mc - m);
            l = fmaf(lc, f, l);
            acc = fmaf(ac, f, acc);
        }
    }
    sm[j][cl] = m;
    sl[j][cl] = l;
    sa[j][cl] = acc;
    __syncthreads();
    if (t < 32) {
        float M = -INFINITY;
        for (int r = 0; r < 32; ++r) M = fmaxf(M, sm[r][t]);
        float ls = 0.0f, as = 0.0f;
        if (M != -INFINITY) {
            for (int r = 0; r < 32; ++r) {
                const float f = __expf(sm[r][t] - M);
                ls = fmaf(sl[r][t], f, ls);
                as = fmaf(sa[r][t], f, as);
            }
        }
        const int b = bkv / H_kv, h = bkv % H_kv;
        out[(int64_t(b) * H_q + h * G + g) * kD + c] = ls > 0.0f ? as / ls : 0.0f;
    }
}

// ---------------------------------------------------------------- debug S view
__global__ __launch_bounds__(256) void seg_compact_kernel(const int32_t *__restrict__ seg_idx,
                                                          const int32_t *__restrict__ seg_cnt,
                                                          int32_t n_chunks, int32_t n,
                                                          int32_t *__restrict__ s_idx,
                                                          int32_t *__restrict__ s_len)
{
    const int bhq = blockIdx.x, t = threadIdx.x;
    int64_t off = 0;
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int cnt = seg_cnt[int64_t(bhq) * n_chunks + ch];
        const int32_t *src = seg_idx + (int64_t(bhq) * n_chunks + ch) * kChunk;
        if (s_idx)
            for (int r = t; r < cnt; r += 256) s_idx[int64_t(bhq) * n + off + r] = src[r];
        off += cnt;
    }
    if (t == 0 && s_len) s_len[bhq] = int32_t(off);
}

// Workgroups of scan_gather_kernel<G, T> resident at once on the current
// device (compute units x workgroups per unit), cached per device.
template <int G, typename T>
int resident_workgroups()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_gather_kernel<G, T>, 256, 0) !=
                hipSuccess)
            return 0;
        cached[dev] = cus * (per_cu > 0 ? per_cu : 1);
    }
    return cached[dev];
}

template <int G, typename T>
hipError_t launch_scan_gather_t(const DecodeArgs &a, hipStream_t s)
{
    const int64_t chunks = int64_t(a.B) * a.H_kv * a.n_chunks;
    const int slots = resident_workgroups<G, T>();
    if (slots <= 0) return hipErrorInvalidDevice;
    const int32_t cpb = ceil_div(chunks, slots);
    const dim3 grid(ceil_div(chunks, cpb));
    if (a.ev_begin || a.ev_end) {
        // timed entry point: the runtime stamps the events at this kernel's
        // own start and end
        hipExtLaunchKernelGGL(scan_gather_kernel<G, T>, grid, dim3(256), 0, s,
                              static_cast<hipEvent_t>(a.ev_begin),
                              static_cast<hipEvent_t>(a.ev_end), 0, a, cpb);
    } else {
        scan_gather_kernel<G, T><<<grid, 256, 0, s>>>(a, cpb);
    }
    return hipGetLastError();
}

template <int G>
hipError_t launch_scan_gather(const DecodeArgs &a, hipStream_t s)
{
    hipError_t e = a.dtype == MP_BF16 ? launch_scan_gather_t<G, uint16_t>(a, s)
                                      : launch_scan_gather_t<G, float>(a, s);
    if (e != hipSuccess) return e;
    merge_kernel<G><<<dim3(a.B * a.H_kv * G, kD / 32), 1024, 0, s>>>(a.part, a.n_chunks, a.H_kv,
                                                                   a.H_q, a.out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    const int BHq = a.B * a.H_q;
    const int TB = a.K > 0 ? 64 / a.K : 64;
    encode_query_kernel<<<dim3(ceil_div(a.L, TB), ceil_div(BHq, 4)), 256, 0, s>>>(
        a.q, BHq, a.W, a.K, a.L, a.qcodes, a.qq, a.qnorm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.G) {
    case 1: e = launch_scan_gather<1>(a, s); break;
    case 2: e = launch_scan_gather<2>(a, s); break;
    case 4: e = launch_scan_gather<4>(a, s); break;
    case 8: e = launch_scan_gather<8>(a, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (a.debug && (a.s_idx || a.s_len)) {
        seg_compact_kernel<<<dim3(BHq), 256, 0, s>>>(a.seg_idx, a.seg_cnt, a.n_chunks, a.n,
                                                     a.s_idx, a.s_len);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace mp
