// tables.hip -- MagicPIG decode through bucketed hash tables on gfx950.
//
// Page "MagicPIG: LSH Sampling for Efficient LLM Generation", Algorithm 1:
// the query's code selects one bucket in each of the L tables, and the keys
// found in at least two of them are the sampled set S; page "MagicPIG: don't
// pick the tallest", section 6 ("The bill"): a table stores a 32-bit token
// index per key, and a query reads about L n / 2^K of them.  The set is the
// one the code scan of decode.hip finds; only the way to it differs.
//
//   build_tables   per (sequence, KV head) unit and table: a counting sort of
//                  the keys by their code (bucket starts + keys grouped by
//                  bucket).  Keys within a bucket come in no fixed order;
//                  nothing downstream depends on it.
//   collide        per query head and slice of its L tables (collide_plan
//                  sets the slices): the query's codes for the slice's
//                  tables unless encode_query has made them, then the
//                  slice's buckets, each key marked in an LDS bitmap of 2
//                  bits (seen once, seen twice), written out per slice.
//   table_gather   per 512-key chunk: the G heads' slice bits of its keys
//                  (seen twice = in one slice, or once in two) give the
//                  sampled / exact list; gather-SNIS as in the code scan
//                  (gather_common.h) writes the chunk's partial softmax, which
//                  the merge of decode.hip combines, or, where a unit has few
//                  chunks (at most 32, or 64 with 32 units or more), the
//                  workgroup that stores a unit's last one merges in this
//                  kernel (store_count_merge; collide zeroes the counts).
#include <hip/hip_ext.h>

#include <algorithm>

#include "gather_common.h"

namespace mp {

namespace {

constexpr int kBuildThreads = 1024;
// LDS of collide_kernel's code step: q (kD floats) and the sign bits of a
// slice's hyperplanes (at most 255 tables of kMaxTableK bits).
constexpr size_t kCollideCodeLds = kD * 4 + 255 * kMaxTableK;

// Exclusive prefix sum of one value per thread over a workgroup of
// kBuildThreads (16 waves); every thread gets its own prefix and the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wtot, uint32_t &total)
{
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wtot[w] = x;
    __syncthreads();
    uint32_t base = 0, all = 0;
    for (int j = 0; j < kBuildThreads / 64; ++j) {
        if (j < w) base += wtot[j];
        all += wtot[j];
    }
    total = all;
    __syncthreads();
    return base + x - v;
}

// Codes of the 16 keys i0 .. i0 + 15 (i0 a multiple of 16) in the table whose
// plane rows start at `pl` (a table's rows recur every chunk_stride words,
// one chunk of 512 keys apart): its K bits per key, one per plane row.  The
// K plane words that hold the 16 keys are loaded once.
__device__ __forceinline__ void key_codes16(const uint32_t *pl, int64_t chunk_stride, int K, int i0,
                                            uint32_t (&c)[16])
{
    const uint32_t *w = pl + int64_t(i0 / kChunk) * chunk_stride + (i0 % kChunk) / 32;
    const int sh = i0 % 32;   // 0 or 16
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = 0u;
    for (int b = 0; b < K; ++b) {
        const uint32_t x = w[b * kWords] >> sh;
#pragma unroll
        for (int k = 0; k < 16; ++k) c[k] |= ((x >> k) & 1u) << b;
    }
}

// Keys per staged tile of the scatter: its entries are grouped by bucket in
// LDS, then written out as one run per bucket (key index and code packed in
// a word: n < 2^20 and K <= 12 where tables are built).
constexpr int kStageTile = 16384;
constexpr int kStageKeys = kStageTile / kBuildThreads;   // per thread
// tables are built only where the collide bitmap (2 bits a key) fits in the
// 160 KB of LDS: n < 160 KB * 4 keys a byte < 2^20
static_assert(int64_t(160 * 1024) * 4 < (int64_t(1) << 20), "key indices must fit in 20 bits");
static_assert(kMaxTableK <= 12, "codes must fit in 12 bits");
static_assert(kStageKeys == 16, "a thread stages the 16 keys whose codes it reads together");

// Block = one (unit, table).  LDS: hist (nbins counters, then cursors), the
// tile's counts and starts per bucket, the staged tile.
__global__ __launch_bounds__(kBuildThreads) void build_tables_kernel(
    const uint32_t *__restrict__ planes, int32_t n, int32_t nc_cap, int32_t L, int32_t K,
    int32_t Kr, int32_t nbins, uint32_t *__restrict__ off, uint32_t *__restrict__ ent)
{
    extern __shared__ uint32_t hist[];
    __shared__ uint32_t wtot[kBuildThreads / 64];
    const int u = blockIdx.x / L, l = blockIdx.x % L;
    const int t = threadIdx.x;
    const int64_t cstride = int64_t(L) * Kr * kWords;
    const uint32_t *pl = planes + int64_t(u) * nc_cap * cstride + int64_t(l) * Kr * kWords;
    for (int b = t; b < nbins; b += kBuildThreads) hist[b] = 0u;
    __syncthreads();
    // 16 consecutive keys a thread: their K plane words are loaded once
    for (int i0 = 16 * t; i0 < n; i0 += 16 * kBuildThreads) {
        uint32_t c[16];
        key_codes16(pl, cstride, K, i0, c);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (i0 + k < n) atomicAdd(&hist[c[k]], 1u);
    }
    __syncthreads();
    // thread t owns bins [t per, (t+1) per)
    const int per = (nbins + kBuildThreads - 1) / kBuildThreads;   // <= 4 for K <= 12
    uint32_t loc[4], sum = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = t * per + k;
        loc[k] = (k < per && b < nbins) ? hist[b] : 0u;
        sum += loc[k];
    }
    uint32_t all;
    uint32_t start = block_exclusive_scan(sum, wtot, all);
    uint32_t *o = off + (int64_t(u) * L + l) * (nbins + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = t * per + k;
        if (k < per && b < nbins) {
            o[b] = start;
            hist[b] = start;
            start += loc[k];
        }
    }
    if (t == 0) o[nbins] = uint32_t(n);
    __syncthreads();
    uint32_t *e = ent + (int64_t(u) * L + l) * n;
    uint32_t *tcount = hist + nbins, *tstart = tcount + nbins, *stage = tstart + nbins;
    for (int t0 = 0; t0 < n; t0 += kStageTile) {
        const int tn = min(kStageTile, n - t0);
        for (int b = t; b < nbins; b += kBuildThreads) tcount[b] = 0u;
        __syncthreads();
        // each key's bucket and its rank among the tile's keys of that bucket
        // thread t takes the tile's keys 16 t .. 16 t + 15
        uint32_t pk[kStageKeys], rk[kStageKeys];
        {
            uint32_t c[16];
            if (16 * t < tn) key_codes16(pl, cstride, K, t0 + 16 * t, c);
#pragma unroll
            for (int k = 0; k < kStageKeys; ++k) {
                const int j = 16 * t + k;
                pk[k] = rk[k] = 0u;
                if (j < tn) {
                    pk[k] = uint32_t(t0 + j) | (c[k] << 20);
                    rk[k] = atomicAdd(&tcount[c[k]], 1u);
                }
            }
        }
        __syncthreads();
        // the tile's start of each bucket (same bin ownership as above)
        uint32_t tl[4], ts = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = t * per + k;
            tl[k] = (k < per && b < nbins) ? tcount[b] : 0u;
            ts += tl[k];
        }
        uint32_t tall;
        uint32_t tb = block_exclusive_scan(ts, wtot, tall);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = t * per + k;
            if (k < per && b < nbins) {
                tstart[b] = tb;
                tb += tl[k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kStageKeys; ++k)
            if (16 * t + k < tn) stage[tstart[pk[k] >> 20] + rk[k]] = pk[k];
        __syncthreads();
        // one run per bucket, consecutive entries to consecutive words
        for (int j = t; j < tn; j += kBuildThreads) {
            const uint32_t v = stage[j], c = v >> 20;
            e[hist[c] + (uint32_t(j) - tstart[c])] = v & 0xFFFFFu;
        }
        __syncthreads();
        for (int b = t; b < nbins; b += kBuildThreads) hist[b] += tcount[b];
        __syncthreads();
    }
}

// Block = one slice of the L tables of one query head (`slices` slices).
// With kOwnCodes, first the head's codes for the slice's tables, computed
// here rather than in a kernel of their own: thread = (hyperplane, quarter of
// the dims), 256 hyperplanes a pass, with the projection of the code scan's
// query encoder (quarter_dot), so both paths find the same codes; the sign
// bits meet in LDS.  The codes also go to qcodes (the debug view) and the
// first slice writes |q|.  Otherwise the codes come from qcodes.  Then the
// bucket walk.  LDS: the slice's bitmap (2 bits per
// key: bit 0 = seen in a bucket, bit 1 = seen in two), then per table of the
// slice the bucket start and the prefix of bucket sizes; the code step uses
// the front of that space before the bitmap is cleared.  The entries of the
// slice's buckets are walked as one flat range, four per thread at a time so
// their loads overlap.  Slice bitmaps go out side by side; the gather
// combines them.
template <bool kOwnCodes>
__global__ __launch_bounds__(kBuildThreads) void collide_kernel(
    const float *__restrict__ q, const float *__restrict__ W, int32_t K,
    const uint32_t *__restrict__ off, const uint32_t *__restrict__ ent, int32_t H_q, int32_t H_kv,
    int32_t n, int32_t nwords, int32_t L, int32_t nbins, uint32_t *__restrict__ bits,
    uint16_t *__restrict__ qcodes, float *__restrict__ qnorm, int32_t slices,
    int32_t *__restrict__ cnt, int32_t ncnt)
{
    extern __shared__ uint32_t sm[];
    __shared__ uint32_t wtot[kBuildThreads / 64];
    if (blockIdx.x == 0)   // the gather's per-unit record counts start at zero
        for (int i = threadIdx.x; i < ncnt; i += kBuildThreads) cnt[i] = 0;
    const int bhq = blockIdx.x / slices, sl = blockIdx.x % slices;
    const int l0 = (sl * L) / slices, nl = ((sl + 1) * L) / slices - l0;
    const int t = threadIdx.x;
    uint32_t code = 0u;
    if (kOwnCodes) {
        // ---- the slice's query codes (the first W rows are loaded before q is
        // staged, so that the two loads overlap)
        float4 *sq4 = reinterpret_cast<float4 *>(sm);              // q: kD / 4 float4
        uint8_t *sbit = reinterpret_cast<uint8_t *>(sm + kD);      // nl * K sign bits
        const int nh = nl * K, hp0 = t >> 2, dq = t & 3;
        constexpr int kPass = kBuildThreads / 4;                   // hyperplanes a pass
        float4 wr[2][8];
        auto load_pass = [&](int p0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hp = p0 + h * kPass + hp0;
                if (hp < nh) {
                    load_w_quarter(wr[h], W + (int64_t(l0) * K + hp) * kD, dq);
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) wr[h][c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
            }
        };
        load_pass(0);
        if (t < kD / 4) sq4[t] = reinterpret_cast<const float4 *>(q + int64_t(bhq) * kD)[t];
        __syncthreads();
        if (sl == 0 && t < 32) {
            const float nrm = norm32(sq4[t]);
            if (t == 0) qnorm[bhq] = nrm;
        }
        for (int p0 = 0; p0 < nh; p0 += 2 * kPass) {
            if (p0 > 0) load_pass(p0);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int hp = p0 + h * kPass + hp0;
                const float sdot = quarter_dot(wr[h], sq4, dq);
                if (dq == 0 && hp < nh) sbit[hp] = sdot > 0.0f ? 1 : 0;
            }
        }
        __syncthreads();
        if (t < nl) {
            for (int bb = 0; bb < K; ++bb) code |= uint32_t(sbit[t * K + bb]) << bb;
            qcodes[int64_t(bhq) * L + l0 + t] = uint16_t(code);
        }
    } else if (t < nl) {
        code = qcodes[int64_t(bhq) * L + l0 + t];
    }
    __syncthreads();   // the code step's LDS is the bitmap's from here on

    // ---- the bucket walk
    uint32_t *bm = sm;
    uint32_t *bstart = sm + nwords;
    uint32_t *bpre = bstart + nl;   // nl + 1 entries
    const int b = bhq / H_q, hq = bhq % H_q, G = H_q / H_kv;
    const int u = b * H_kv + hq / G;
    for (int i = t; i < nwords; i += kBuildThreads) bm[i] = 0u;
    uint32_t size = 0u;
    if (t < nl) {
        const uint32_t *o = off + (int64_t(u) * L + l0 + t) * (nbins + 1);
        const uint32_t s0 = o[code];
        bstart[t] = s0;
        size = o[code + 1] - s0;
    }
    uint32_t total;
    const uint32_t pre = block_exclusive_scan(size, wtot, total);
    if (t < nl) bpre[t] = pre;
    if (t == 0) bpre[nl] = total;
    __syncthreads();
    const uint32_t *eu = ent + (int64_t(u) * L + l0) * n;
    for (uint32_t base = t; base < total; base += 4 * kBuildThreads) {
        uint32_t key[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t idx = base + k * kBuildThreads;
            key[k] = 0xFFFFFFFFu;
            if (idx < total) {
                int lo = 0, hi = nl - 1;   // last table whose prefix is <= idx
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (bpre[mid] <= idx) lo = mid;
                    else hi = mid - 1;
                }
                key[k] = eu[int64_t(lo) * n + bstart[lo] + (idx - bpre[lo])];
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (key[k] == 0xFFFFFFFFu) continue;
            const uint32_t w = key[k] >> 4, one = 1u << (2 * (key[k] & 15u));
            if (atomicOr(&bm[w], one) & one) atomicOr(&bm[w], one << 1);
        }
    }
    __syncthreads();
    uint32_t *ob = bits + int64_t(bhq) * slices * nwords + sl * nwords;
    for (int i = t; i < nwords; i += kBuildThreads) ob[i] = bm[i];
}

// Waves per SIMD the register budget is cut for: with bf16 rows 5 up to
// G = 4 (more chunks resident at once; the second gather round then loads its
// rows when it starts) and 4 at G = 8 (the second round's rows issued ahead);
// with fp32 rows what the registers give (LDS holds it to 4 or fewer).
template <int G, typename T>
constexpr int table_occupancy() { return sizeof(T) == 2 ? (G <= 4 ? 5 : 4) : 2; }
template <int G, typename T>
constexpr bool table_rows_ahead() { return sizeof(T) == 2 && G > 4; }

// Block = one 512-key chunk of one unit and its G query heads; S slice
// bitmaps per head (a compile-time count, so that their loads issue together).
template <int G, typename T, int S>
__global__ __launch_bounds__(256, (table_occupancy<G, T>())) void table_gather_kernel(DecodeArgs a,
                                                                                     int32_t nwords,
                                                                                     int32_t frec)
{
    __shared__ uint32_t ulist[kChunk];
    __shared__ int wsum[4];
    __shared__ __align__(16) float sq[G][kD];
    __shared__ float sqn[2 * G + 1];   // |q_g|, q_g.mu, the lift radius
    __shared__ __align__(16) float smu[kD];
    __shared__ GatherLds<G, T> gl;
    // Workgroup b takes unit b % units and, counting back from the unit's
    // end, chunk b / units: each sequence's last chunk (its exact local
    // window, the longest list) goes to the workgroups dispatched first.
    const int units = a.B * a.H_kv;
    const int bkv = blockIdx.x % units, chunk = a.n_chunks - 1 - blockIdx.x / units;
    const int bhq0 = (bkv / a.H_kv) * a.H_q + (bkv % a.H_kv) * G;
    const int t = threadIdx.x, gi = t >> 4, li = t & 15;
    // Thread t owns keys 2t and 2t+1: one 4-bit field of a bitmap word.
    const int n = a.n;
    const int64_t key0 = int64_t(chunk) * kChunk + 2 * t;
    const int word = int(key0 >> 4), sh = 2 * int(key0 & 15);

    // Every load of the prologue (queries, norms, lift radius, mean, the
    // slice bitmaps) is issued before any of them is waited for: one round
    // trip, not one per LDS store.
    constexpr int kQ = (G * kD + 255) / 256;
    float qv[kQ];
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
        const int i = t + 256 * j;
        qv[j] = i < G * kD ? a.q[int64_t(bhq0) * kD + i] : 0.0f;
    }
    const float qn = t < G ? a.qnorm[bhq0 + t] : 0.0f;
    const float rn = t == 0 && a.rnorm ? a.rnorm[bkv] : 0.0f;
    const float mv = t < kD ? a.mu[int64_t(bkv) * kD + t] : 0.0f;
    uint32_t fb[G][S];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int sl = 0; sl < S; ++sl)
            fb[g][sl] = a.bits[(int64_t(bhq0 + g) * S + sl) * nwords + word];
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
        const int i = t + 256 * j;
        if (i < G * kD) sq[i / kD][i % kD] = qv[j];
    }
    if (t < G) sqn[t] = qn;
    if (t == 0) sqn[2 * G] = rn;
    if (t < kD) smu[t] = mv;

    uint32_t hm[2] = {0u, 0u}, c2[2][G];
    bool ex[2], fl[2];
    uint32_t once[G], twice[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        // Seen twice: in one slice, or once in each of two slices.  The
        // slices are merged whole words at a time, 16 keys of (twice, once)
        // bit pairs: once = once_a | once_b, twice = twice_a | twice_b |
        // (once_a & once_b), the last term moved up from the once bit.
        uint32_t m = fb[g][0];
#pragma unroll
        for (int sl = 1; sl < S; ++sl) {
            const uint32_t b = fb[g][sl];
            m = ((m & b & 0x55555555u) << 1) | (m | b);
        }
        const uint32_t f = m >> sh;   // this thread's 2 keys x 2 bits
        once[g] = f & 0x5u;
        twice[g] = (f >> 1) & 0x5u;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int64_t i = key0 + e;
        const bool valid = i < n;
        ex[e] = valid && (i < a.n_sink || i >= int64_t(n) - a.n_local);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            c2[e][g] = ((twice[g] >> (2 * e)) & 1u) ? 2u : ((once[g] >> (2 * e)) & 1u);
            if (valid && !ex[e] && c2[e][g] == 2u) hm[e] |= 1u << g;
        }
        fl[e] = ex[e] || hm[e] != 0u;
    }
    const int total = compact_list(
        fl[0], fl[1], uint32_t(2 * t) | (hm[0] << 16) | (uint32_t(ex[0]) << 24),
        uint32_t(2 * t + 1) | (hm[1] << 16) | (uint32_t(ex[1]) << 24), ulist, wsum, t);
    if (a.debug) {
        if (a.counts) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (key0 + e < n)
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        a.counts[int64_t(bhq0 + g) * n + key0 + e] = uint8_t(c2[e][g]);
        }
        write_seg_lists<G>(a, hm[0], hm[1], key0, bhq0, chunk, wsum, t);
    }
    stage_qmu<G>(sq, smu, sqn, t);   // the staged queries are visible past the compaction's barriers
    __syncthreads();   // ulist, the staged queries and q.mu complete

    typename Row8<T>::raw kr[kRowsPerGroup], vr[kRowsPerGroup];
    const T *kb, *vb;
    row_bases<T>(a, bkv, li, kb, vb);
    load_rows<T>(a, kb, vb, ulist, 0, min(kRound, total), chunk, gi, kr, vr);
    GatherAcc<G> acc;
    acc.reset();
    gather_chunk_into<G, T, table_rows_ahead<G, T>()>(a, gl, ulist, total, chunk, bkv, sq, sqn, smu,
                                                       kr, vr, acc, t, gi, li);
    if (frec > 0)   // few chunks a unit: the unit's last merges its records here
        store_count_merge<G, T, kFusedMergeWide>(a, acc, chunk, bkv, frec, gl, wsum, t);
    else
        gather_store<G>(a, acc, chunk, bkv, t);
}

template <int G, typename T, int S>
hipError_t launch_table_gather_t(const DecodeArgs &a, int32_t nwords, hipStream_t s)
{
    const dim3 grid(a.B * a.H_kv * a.n_chunks);
    return launch_timed(table_gather_kernel<G, T, S>, grid, dim3(256), 0, s, a.ev_begin, a.ev_end,
                        a, nwords, fused_merge_records(a, G, 1, kFusedMergeWide));
}

template <int G, int S>
hipError_t launch_table_gather_s(const DecodeArgs &a, int32_t nwords, hipStream_t s)
{
    return a.dtype == MP_BF16 ? launch_table_gather_t<G, uint16_t, S>(a, nwords, s)
                              : launch_table_gather_t<G, float, S>(a, nwords, s);
}

template <int G>
hipError_t launch_table_gather(const DecodeArgs &a, int32_t nwords, int32_t slices, hipStream_t s)
{
    switch (slices) {
    case 4: return launch_table_gather_s<G, 4>(a, nwords, s);
    case 8: return launch_table_gather_s<G, 8>(a, nwords, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Dynamic LDS of build_tables_kernel: 3 x 2^K bucket words and the staged tile.
static size_t build_tables_lds(int K) { return (size_t(3) * (size_t(1) << K) + kStageTile) * 4; }

hipError_t launch_build_tables(const mp_index_impl &idx, hipStream_t s)
{
    static PerDevice attr;
    hipError_t e = attr.once([](int) {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(build_tables_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   int(build_tables_lds(kMaxTableK)));
    });
    if (e != hipSuccess) return e;
    const IndexLayout &lay = idx.lay;
    const int nbins = 1 << lay.K;
    return launch(build_tables_kernel, dim3(lay.B * lay.H_kv * lay.L), dim3(kBuildThreads),
                  build_tables_lds(lay.K), s, static_cast<const uint32_t *>(idx.planes), lay.n,
                  lay.nc_cap, lay.L, lay.K, lay.Kr, nbins, idx.tab_off, idx.tab_ent);
}

hipError_t launch_decode_tables(const DecodeArgs &a, hipStream_t s)
{
    const CollidePlan plan = collide_plan(int64_t(a.B) * a.H_q);
    hipError_t e = plan.own_codes ? hipSuccess : launch_encode_query(a, s);
    if (e != hipSuccess) return e;
    static PerDevice attr;
    e = attr.once([](int) {
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(collide_kernel<true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           int(kCollideLdsMax));
        if (r != hipSuccess) return r;
        return hipFuncSetAttribute(reinterpret_cast<const void *>(collide_kernel<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(kCollideLdsMax));
    });
    if (e != hipSuccess) return e;
    const int32_t n_pad = a.n_chunks * kChunk, nwords = n_pad / 16;
    // bounds any slice; at least the code step's q and sign bits
    const size_t lds = std::max(size_t(nwords) * 4 + size_t(2 * a.L + 1) * 4, kCollideCodeLds);
    e = launch(plan.own_codes ? collide_kernel<true> : collide_kernel<false>,
               dim3(a.B * a.H_q * plan.slices), dim3(kBuildThreads), lds, s, a.q, a.W, a.K,
               static_cast<const uint32_t *>(a.tab_off), static_cast<const uint32_t *>(a.tab_ent),
               a.H_q, a.H_kv, a.n, nwords, a.L, 1 << a.K, a.bits, a.qcodes, a.qnorm, plan.slices,
               a.unit_cnt, a.unit_cnt ? a.B * a.H_kv : 0);
    if (e != hipSuccess) return e;
    switch (a.G) {
    case 1: e = launch_table_gather<1>(a, nwords, plan.slices, s); break;
    case 2: e = launch_table_gather<2>(a, nwords, plan.slices, s); break;
    case 4: e = launch_table_gather<4>(a, nwords, plan.slices, s); break;
    case 8: e = launch_table_gather<8>(a, nwords, plan.slices, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // a record per chunk, merged inside table_gather where a unit has few
    if (fused_merge_records(a, a.G, 1, kFusedMergeWide) == 0 &&
        (e = launch_merge(a, 1, s)) != hipSuccess)
        return e;
    return launch_seg_compact(a, s);
}

}  // namespace mp
