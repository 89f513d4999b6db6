// decode.hip -- one MagicPIG decode step on gfx950: two or three launches.
//
//   encode_query   SimHash codes of the raw queries (page "MagicPIG: LSH
//                  Sampling for Efficient LLM Generation", algorithm steps:
//                  the query's code from the shared projector).
//   scan_gather    a workgroup takes a run of 512-key chunks (each of one KV
//                  head and its G query heads), no more workgroups than are
//                  resident at once (at most two a CU up to G = 4); per chunk:
//                  (a) stream the chunk's code planes and mark, per key and
//                      query head, whether the key shares the query's bucket
//                      in at least one and in at least two tables (32 keys per
//                      32-bit word: a key matches a table iff each of its K
//                      plane bits equals the query's bit);
//                  (b) a key is sampled for a head iff that count is >= 2 and
//                      the key is not in the exact set T (method details and
//                      page "MagicPIG: don't pick the tallest", section 5);
//                      ballot/prefix-sum compaction of the union of sampled
//                      and exact keys into an ascending LDS list;
//                  (c) gather the listed K/V rows, recompute q.k and the cosine
//                      to the centered key, u_i = P[Binomial(L, p^K) >= 2],
//                      z = q.k*scale - log u (z = q.k*scale on T), and run an
//                      online softmax per query head (algorithm steps: one
//                      softmax over [w_S, w_T]/sqrt(d) - log[u, 1]) that
//                      carries on over the run's chunks of one unit; the
//                      partial softmax (max, sum, unnormalised accumulator)
//                      per head goes to scratch, one record a run and unit.
//                  The code stream runs two batches ahead across chunks, and
//                  (c) runs one chunk late, so a chunk's rows arrive while the
//                  next chunk is scanned.
//   counts         (debug only) the exact collision count of every key and
//                  query head, from the planes.
//   merge          log-sum-exp merge of the partial records of every query head
//                  (system co-design: partial attention outputs are merged
//                  recursively).  Where a unit has at most 32 records it runs
//                  inside scan_gather instead (gather_common.h,
//                  store_count_merge): records go out with device-scope
//                  stores and the workgroup that counts a unit's last one
//                  merges them.  Otherwise a kernel of its own, whose launch
//                  boundary makes the records of blocks on other XCDs visible
//                  (one workgroup reading a unit's many records would lengthen
//                  the scan's tail more than the launch costs).
#include <hip/hip_ext.h>
#include <math.h>

#include "append_codes.h"
#include "gather_common.h"

namespace mp {
namespace {

// Table slots of a workgroup: thread t scans word t % kWords of the chunk in
// tables t / kWords, + kSlots, ...
constexpr int kSlots = 256 / kWords;
#ifndef MP_SCAN_TB
#define MP_SCAN_TB 1
#endif
constexpr int kTB = MP_SCAN_TB;   // tables per plane batch of a thread

// Bit b of x, replicated over 32 bits (0 or ~0).
__device__ __forceinline__ uint32_t bit_mask(uint32_t x, int b)
{
    return uint32_t(__builtin_amdgcn_sbfe(int32_t(x), uint32_t(b), 1u));
}

// Fourth word of a raw buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// acc & ~(p ^ m) in one v_bitop3_b32 (truth table over (p, acc, m): set where
// acc = 1 and p = m).  The compiler splits this form into XOR and OR3.
__device__ __forceinline__ uint32_t and_xnor(uint32_t acc, uint32_t p, uint32_t m)
{
    uint32_t d;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x84" : "=v"(d) : "v"(p), "v"(acc), "v"(m));
    return d;
}

// ---------------------------------------------------------------- query codes
// Block: TB = 64/K whole tables (<= 64 hyperplanes) x QH query heads.
// Thread = (hyperplane, quarter of the dims): four lanes read one W row
// together (64 contiguous bytes a load) and keep their 32 dims in registers
// for all the block's heads, whose queries are LDS broadcasts; two shuffles
// add the quarters.  Sign bits meet in LDS and are packed per (head, table).
// QH = 2 up to 32 query heads (twice the blocks, each with half the dots:
// the step 0.2-0.3 us shorter at 16K and 96K), 4 beyond (2 was 2.3 us longer
// at batch 16, 6,400 blocks).
template <int QH>
__device__ __forceinline__ void encode_query_block(const float *__restrict__ q, int32_t BHq,
                                                   const float *__restrict__ W, int32_t K,
                                                   int32_t L, uint16_t *__restrict__ qcodes,
                                                   uint32_t *__restrict__ qq,
                                                   float *__restrict__ qnorm, int bx, int by,
                                                   float4 (*sQ)[kD / 4], uint8_t (*sbit)[64],
                                                   int t)
{
    const int hp = t >> 2, dq = t & 3;
    const int TB = K > 0 ? 64 / K : 64;
    const int l0 = bx * TB;
    const int nt = min(TB, L - l0);
    const int nh = nt * K;
    const int q0 = by * QH;
    const int nq = min(QH, BHq - q0);
    const float4 *q4 = reinterpret_cast<const float4 *>(q + int64_t(q0) * kD);
    if (t < nq * (kD / 4)) sQ[t / (kD / 4)][t % (kD / 4)] = q4[t];
    float4 wr[8];
    if (hp < nh) {
        load_w_quarter(wr, W + (int64_t(l0) * K + hp) * kD, dq);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) wr[c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    __syncthreads();
    if (bx == 0) {                 // |q| of the block's heads, for the cosines
        const int j = t >> 5, c4 = t & 31;
        const float nrm = norm32(j < nq ? sQ[j][c4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        if (j < nq && c4 == 0) qnorm[q0 + j] = nrm;
    }
    for (int j = 0; j < nq; ++j) {
        const float sdot = quarter_dot(wr, sQ[j], dq);
        if (dq == 0 && hp < nh) sbit[j][hp] = sdot > 0.0f ? 1 : 0;
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

// Encode blocks over a 1-D grid: (table block bx < nbx, head block by < nby)
// of block b.  Workgroups go to the 8 XCDs round-robin by index, so the
// blocks of one table block (the same W rows, for every head block) are
// placed on one XCD, b % 8 = bx % 8, and read those rows into its L2 once
// instead of on every XCD.  The grid then has 8 nby ceil(nbx / 8) blocks;
// those with bx >= nbx have nothing to do.
inline int encode_grid(int nbx, int nby) { return 8 * nby * ((nbx + 7) / 8); }
__device__ __forceinline__ bool encode_coords(int b, int nbx, int nby, int &bx, int &by)
{
    const int k = b / 8;
    by = k % nby;
    bx = 8 * (k / nby) + b % 8;
    return bx < nbx;
}

template <int QH>
__global__ __launch_bounds__(256) void encode_query_kernel(const float *__restrict__ q,
                                                           int32_t BHq,
                                                           const float *__restrict__ W, int32_t K,
                                                           int32_t L,
                                                           uint16_t *__restrict__ qcodes,
                                                           uint32_t *__restrict__ qq,
                                                           float *__restrict__ qnorm, int32_t nbx,
                                                           int32_t nby, int32_t *__restrict__ cnt,
                                                           int32_t ncnt)
{
    __shared__ float4 sQ[QH][kD / 4];
    __shared__ uint8_t sbit[QH][64];
    if (blockIdx.x == 0)   // the scan's per-unit record counts start at zero
        for (int i = threadIdx.x; i < ncnt; i += 256) cnt[i] = 0;
    int bx, by;
    if (!encode_coords(blockIdx.x, nbx, nby, bx, by)) return;   // the whole block
    encode_query_block<QH>(q, BHq, W, K, L, qcodes, qq, qnorm, bx, by, sQ, sbit, threadIdx.x);
}

// The query encode and an append of a few keys (append_codes.h) in one
// launch, for a decode that first grows its index: blocks [0, n_enc) are the
// encode blocks (encode_coords), the rest the append's blocks (unit,
// hyperplane block of kAppendRows).  The two write disjoint memory; the scan
// that reads both comes after the launch.
template <int QH, typename T>
__global__ __launch_bounds__(256) void encode_append_kernel(
    const float *__restrict__ q, int32_t BHq, const float *__restrict__ W, int32_t K, int32_t L,
    uint16_t *__restrict__ qcodes, uint32_t *__restrict__ qq, float *__restrict__ qnorm,
    int32_t nbx, int32_t nby, int32_t n_enc, const T *__restrict__ keys, int64_t sb, int64_t sh,
    int64_t sn, int32_t H, int32_t n0, int32_t n1, int32_t nc_cap, const float *__restrict__ mu,
    uint32_t *__restrict__ planes, int32_t nhb, int32_t *__restrict__ cnt, int32_t ncnt)
{
    __shared__ __align__(16) float sx[kAppendMax][kD];   // the encode's LDS is carved from it
    static_assert(QH * (kD / 4) * 16 + QH * 64 <= sizeof(sx), "encode LDS fits");
    const int b = blockIdx.x, t = threadIdx.x;
    if (b == 0)   // the scan's per-unit record counts start at zero
        for (int i = t; i < ncnt; i += 256) cnt[i] = 0;
    if (b < n_enc) {
        float4(*sQ)[kD / 4] = reinterpret_cast<float4(*)[kD / 4]>(&sx[0][0]);
        uint8_t(*sbit)[64] = reinterpret_cast<uint8_t(*)[64]>(&sx[QH][0]);
        int bx, by;
        if (encode_coords(b, nbx, nby, bx, by))   // uniform over the block
            encode_query_block<QH>(q, BHq, W, K, L, qcodes, qq, qnorm, bx, by, sQ, sbit, t);
    } else {
        const int ab = b - n_enc;
        append_codes_block<T>(keys, sb, sh, sn, H, n0, n1, nc_cap, mu, W, K, L, planes, ab / nhb,
                              ab % nhb, t, sx);
    }
}

// ---------------------------------------------------------------- scan + gather
// Waves per SIMD the register budget is cut for: 3 up to G = 4 with bf16 rows
// (the next chunk's first plane batches stay in registers through a gather),
// 2 otherwise.
#ifndef MP_SCAN_OCC
#define MP_SCAN_OCC 3
#endif
template <int G, typename T>
constexpr int scan_occupancy() { return G <= 2 || (G == 4 && sizeof(T) == 2) ? MP_SCAN_OCC : 2; }

// Plane rows loaded per table: Kr rounded up to one of a few compiled widths
// (rows past Kr re-read row Kr - 1, which changes nothing).
inline int plane_rows_class(int Kr)
{
    return Kr <= 4 ? 4 : Kr <= 8 ? 8 : Kr <= 9 ? 9 : Kr <= 10 ? 10 : Kr <= 12 ? 12 : 16;
}

// One workgroup takes a run of `cpb` consecutive 512-key chunks (numbered
// over (sequence, KV head) units, then chunks); runs are as equal as the
// chunk count allows and the grid is no larger than what is resident at
// once (resident_workgroups).  Per chunk:
//   (a) scan: thread t takes the 32-key word t % 16 of the chunk in tables
//       t / 16, t / 16 + 16, ...  For each table and query head, the key
//       matches iff its K plane bits equal the query's code bits: an AND of
//       K XNORs per 32 keys.  Per head the thread keeps two masks, "matched
//       at least once" and "at least twice"; the 16 threads of a word merge
//       theirs through LDS atomics;
//   (b) the union of sampled and exact keys is compacted into an ascending
//       LDS list, and the K/V rows of its first kRound entries are loaded;
//   (c) gather-SNIS over the list, run one chunk late, when the rows have
//       long arrived: with bf16 rows the first round's dots and z inside the
//       next chunk's scan and the rest after it, with fp32 rows all of it
//       after the scan.  The chunk folds into the run's partial softmax of its
//       unit, which goes to `part` when the unit's chunks of the run end.
// Each thread reads its tables of all chunks of the run as one stream, one
// table (KP plane words) per batch, in two alternating register buffers
// issued two batches ahead across chunk boundaries.  Every load on the main
// path is unconditional (padding batches and rows re-read an address already
// read and count nothing), so the compiler can wait on each buffer alone
// rather than on every load in flight.
template <int G, typename T, int KP>
__global__ __launch_bounds__(256, (scan_occupancy<G, T>())) void scan_gather_kernel(DecodeArgs a,
                                                                                    int32_t cpb,
                                                                                    int32_t frec)
{
    __shared__ uint32_t seen[2][G][kWords];  // per head and word: matched once / twice
    __shared__ __align__(16) uint32_t sqq[256][G];   // query codes, code | code << 16
    __shared__ uint32_t ulist[kChunk];       // key | headmask << 16 | exact << 24
    __shared__ int wsum[4];
    __shared__ __align__(16) float sq[2][G][kD];   // per staged unit: the group's queries
    __shared__ float sqn[2][2 * G + 1];      // their norms, q_g.mu, the lift radius
    __shared__ __align__(16) float smu[2][kD];   // mean of the unit's keys
    __shared__ GatherLds<G, T> gl;           // one gather round

    const int L = a.L, Kr = a.Kr;
    constexpr bool kSplitGather = sizeof(T) == 2;
    // Where runs align with units, workgroup b takes unit b % units and,
    // counting from the unit's end, its run b / units: the runs that hold a
    // sequence's last chunk (its exact local window, the longest list) go
    // to the workgroups dispatched first, which the wave scheduler, oldest
    // first, serves first.  Otherwise runs are in order.
    int run = blockIdx.x;
    if (a.n_chunks % cpb == 0) {
        const int units = a.B * a.H_kv, per_unit = a.n_chunks / cpb;
        run = (run % units) * per_unit + (per_unit - 1 - run / units);
    }
    const int gc_begin = run * cpb;
    const int nrun = min(cpb, a.B * a.H_kv * a.n_chunks - gc_begin);
    // batches per chunk for every thread: even, and at least 2
    const int nt = (L + kSlots - 1) / kSlots;
    const int nb = uniform(max(2, ((nt + kTB - 1) / kTB + 1) & ~1));
    const int64_t rows_per_chunk = int64_t(L) * Kr * kWords;

    // ---- the plane stream: next batch to load is batch ls of chunk lc of the run ----
    uint32_t bufA[kTB][KP], bufB[kTB][KP];
    const int sslot = threadIdx.x / kWords, sword = threadIdx.x % kWords;
    int lc = 0, ls = 0;
    auto load_next = [&](uint32_t(&buf)[kTB][KP]) {
        const bool past = lc >= nrun;                     // beyond the run: re-read the last batch
        const int c = past ? nrun - 1 : lc, sb = past ? nb - 1 : ls;
        // Raw buffer loads over the chunk's planes: the row offset is an
        // SGPR and the lane's offset one VGPR, so a load costs no VALU.
        const int gcx = gc_begin + c, ubkv = gcx / a.n_chunks;
        const int64_t pchunk = int64_t(ubkv) * a.nc_cap + (gcx - ubkv * a.n_chunks);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(a.planes + pchunk * rows_per_chunk), 0, 0x7FFFFFFF, kBufferWord3);
#pragma unroll
        for (int u = 0; u < kTB; ++u) {
            const int l = min(sslot + (sb * kTB + u) * kSlots, L - 1);
            const uint32_t off = uint32_t(l * Kr * kWords + sword) * 4u;
#pragma unroll
            for (int r = 0; r < KP; ++r)
                buf[u][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, min(r, Kr - 1) * (kWords * 4), 0);
        }
        if (++ls == nb) {
            ls = 0;
            ++lc;
        }
    };
    // A new (sequence, KV head) unit: its query codes for the scan
    // ([table][head]) and, in the other slot, the queries, norms and mean
    // for its gathers (a pending chunk still reads the current slot).  All
    // loads are issued before the first LDS write, so a unit costs one round
    // trip (L <= 255: at most G code words a thread).  q_g.mu follows after
    // the next barrier.
    int cur_unit = -1, slot = 1;
    bool qmu_due = false;
    auto stage_unit = [&](int bkv, int bhq0, int t) {
        slot ^= 1;
        constexpr int kQ = (G * kD + 255) / 256;
        uint32_t qqv[G];
        float qv[kQ];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int i = t + 256 * j;
            qqv[j] = i < G * L ? a.qq[int64_t(bhq0) * L + i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
            const int i = t + 256 * j;
            qv[j] = i < G * kD ? a.q[int64_t(bhq0) * kD + i] : 0.0f;
        }
        const float qn = t < G ? a.qnorm[bhq0 + t] : 0.0f;
        const float rn = t == 0 && a.rnorm ? a.rnorm[bkv] : 0.0f;
        const float mv = t < kD ? a.mu[int64_t(bkv) * kD + t] : 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int i = t + 256 * j;
            if (i < G * L) sqq[i % L][i / L] = qqv[j];
        }
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
            const int i = t + 256 * j;
            if (i < G * kD) sq[slot][i / kD][i % kD] = qv[j];
        }
        if (t < G) sqn[slot][t] = qn;
        if (t == 0) sqn[slot][2 * G] = rn;
        if (t < kD) smu[slot][t] = mv;
        cur_unit = bkv;
        qmu_due = true;
    };

    load_next(bufA);
    load_next(bufB);
    {   // the first unit, its loads in flight with the first two batches
        const int t = threadIdx.x, bkv = gc_begin / a.n_chunks;
        stage_unit(bkv, (bkv / a.H_kv) * a.H_q + (bkv % a.H_kv) * G, t);
    }
    // Wait for both here (only the staging was in flight besides), so that
    // at the top of the chunk loop only the steady-state order of loads is
    // possible: bufA, bufB, then the previous chunk's rows.
#pragma unroll
    for (int u = 0; u < kTB; ++u)
#pragma unroll
        for (int r = 0; r < KP; ++r) asm volatile("" ::"v"(bufA[u][r]), "v"(bufB[u][r]));

    // the chunk whose gather is pending, and its rows
    bool pend = false;
    int p_bkv = 0, p_chunk = 0, p_total = 0, p_slot = 0;
    typename Row8<T>::raw kraw[kRowsPerGroup], vraw[kRowsPerGroup];
    // The run's chunks of one unit fold into one partial softmax, stored as
    // record run - first run of the unit (the merge reads those records).
    GatherAcc<G> acc;
    acc.reset();
    auto store_unit = [&](int ubkv, int t) {
        gather_store<G>(a, acc, run - (ubkv * a.n_chunks) / cpb, ubkv, t);
        acc.reset();
    };

#pragma unroll 1
    for (int it = 0; it < nrun; ++it) {
        // Per-thread offsets are recomputed each chunk from an opaque copy
        // of the thread index: hoisted out of the loop they would hold
        // registers through it.
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int gi = t >> 4, li = t & 15;
        const int gc = gc_begin + it;
        const int bkv = gc / a.n_chunks;
        const int chunk = gc - bkv * a.n_chunks;
        const int bhq0 = (bkv / a.H_kv) * a.H_q + (bkv % a.H_kv) * G;
        const bool staged = bkv != cur_unit;
        if (staged) stage_unit(bkv, bhq0, t);
        if (t < 2 * G * kWords) (&seen[0][0][0])[t] = 0u;
        __syncthreads();
        if (qmu_due) stage_qmu<G>(sq[slot], smu[slot], sqn[slot], t);   // read by the unit's gathers
        qmu_due = false;

        // ---- (a) collision masks ----
        const int tslot = t / kWords, tword = t % kWords;
        uint32_t once[G], twice[G];
#pragma unroll
        for (int g = 0; g < G; ++g) once[g] = twice[g] = 0u;
        auto count_batch = [&](const uint32_t(&buf)[kTB][KP], int sb) {
#pragma unroll
            for (int u = 0; u < kTB; ++u) {
                const int l = tslot + (sb * kTB + u) * kSlots;
                const uint32_t live = l < L ? ~0u : 0u;   // padding tables match nothing
                const int lu = min(l, L - 1);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint32_t qv = sqq[lu][g];
                    uint32_t eq = live;
#pragma unroll
                    for (int r = 0; r < KP; ++r)
                        eq = and_xnor(eq, buf[u][r], bit_mask(qv, min(r, Kr - 1)));
                    twice[g] |= once[g] & eq;
                    once[g] |= eq;
                }
            }
        };
        // The first pair is peeled: entering it, the previous chunk's
        // round-0 rows are younger than bufA and bufB and need not be
        // waited for; inside the loop only the other buffer is younger.
        count_batch(bufA, 0);
        load_next(bufA);
        count_batch(bufB, 1);
        load_next(bufB);
        // ---- (c), first part (bf16 rows): c1 and z of the pending chunk's
        // first round, wave-local, while the two batches just issued are in
        // flight (its rows were loaded before this scan and are older than
        // those batches).  With fp32 rows the registers this needs would
        // cost a wave per SIMD, and the gather runs whole after the scan.
        if (kSplitGather) {
            if (pend)
                gather_head<G, T>(a, gl, ulist, p_total, sq[p_slot], sqn[p_slot], smu[p_slot],
                                  kraw, vraw, gi, li);
            else
                retire_rows<T>(kraw, vraw);   // nothing in flight: returns at once
        }
        for (int sb = 2; sb < nb; sb += 2) {
            count_batch(bufA, sb);
            load_next(bufA);
            count_batch(bufB, sb + 1);
            load_next(bufB);
        }
        // Merge the 16 slots of each word: a key is seen twice if some
        // slot saw it twice or two slots saw it once.
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t before = atomicOr(&seen[0][g][tword], once[g]);
            atomicOr(&seen[1][g][tword], twice[g] | (once[g] & before));
        }

        if (kSplitGather) {
            // the masks in seen are complete, and so is the pending chunk's z
            __syncthreads();
            if (pend) {
                // ---- (c), the rest: c2 of the first round, later rounds;
                // then the pending chunk's list and LDS are free
                gather_tail<G, T>(a, gl, ulist, p_total, p_chunk, p_bkv, sq[p_slot],
                                  sqn[p_slot], smu[p_slot], acc, t, gi, li);
                if (p_bkv != bkv) store_unit(p_bkv, t);   // its unit ends in this run
                __syncthreads();
            }
        } else {
            if (pend) {   // ---- (c) gather-SNIS of the pending chunk
                gather_chunk_into<G, T, false>(a, gl, ulist, p_total, p_chunk, p_bkv, sq[p_slot],
                                               sqn[p_slot], smu[p_slot], kraw, vraw, acc, t, gi,
                                               li);
                if (p_bkv != bkv) store_unit(p_bkv, t);
            } else {
                retire_rows<T>(kraw, vraw);   // nothing in flight: returns at once
            }
            // the masks in seen are complete; the pending chunk's list is no
            // longer read
            __syncthreads();
        }

        // ---- (b) sampled / exact sets and ascending compaction ----
        // Thread t owns keys 2t and 2t+1 of the chunk: bits 2(t%16), +1 of
        // word t/16.
        const int n = a.n;
        const int64_t key0 = int64_t(chunk) * kChunk + 2 * t;
        const int kw = t >> 4, ksh = 2 * (t & 15);
        uint32_t hm[2] = {0u, 0u};
        bool ex[2], fl[2];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t f = seen[1][g][kw] >> ksh;
            hm[0] |= (f & 1u) << g;
            hm[1] |= ((f >> 1) & 1u) << g;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t i = key0 + e;
            const bool valid = i < n;
            ex[e] = valid && (i < a.n_sink || i >= int64_t(n) - a.n_local);
            if (!valid || ex[e]) hm[e] = 0u;
            fl[e] = ex[e] || hm[e] != 0u;
        }
        const int total = compact_list(
            fl[0], fl[1], uint32_t(2 * t) | (hm[0] << 16) | (uint32_t(ex[0]) << 24),
            uint32_t(2 * t + 1) | (hm[1] << 16) | (uint32_t(ex[1]) << 24), ulist, wsum, t);
        if (a.debug) write_seg_lists<G>(a, hm[0], hm[1], key0, bhq0, chunk, wsum, t);
        __syncthreads();   // ulist complete

        // Round 0's rows of this chunk, in flight during the next scan.
        {
            const T *kb, *vb;
            row_bases<T>(a, bkv, li, kb, vb);
            load_rows<T>(a, kb, vb, ulist, 0, min(kRound, total), chunk, gi, kraw, vraw);
        }
        pend = true;
        p_bkv = bkv;
        p_chunk = chunk;
        p_total = total;
        p_slot = slot;
    }

    // The run's last chunk.  Its gather has its own copy here, after the
    // loop, so that inside the loop every path to a gather has come through
    // a scan: there the rows are older than the plane batches in flight, and
    // reading them does not wait for those batches (the compiler merges its
    // count of loads in flight over the paths that meet).  Here the rows are
    // the youngest loads.
    retire_rows<T>(kraw, vraw);
    if (pend) {
        const int t = threadIdx.x;
        // the plane buffers are dead here: the second round's rows go ahead
        // (bf16 rows; fp32 rows would not fit the registers)
        gather_chunk_into<G, T, sizeof(T) == 2>(a, gl, ulist, p_total, p_chunk, p_bkv,
                                                sq[p_slot], sqn[p_slot], smu[p_slot], kraw, vraw,
                                                acc, t, t >> 4, t & 15);
        if (frec > 0)   // runs aligned with units: this run's one record, merged here
            store_count_merge<G, T, kFusedMergeMax>(a, acc, run - (p_bkv * a.n_chunks) / cpb,
                                                    p_bkv, frec, gl, wsum, t);
        else
            store_unit(p_bkv, t);
    }
}

// ---------------------------------------------------------------- debug counts
// Block = one 512-key chunk of one unit; thread t = keys 2t, 2t+1.  For each
// table the two codes are read back from the planes and compared with the
// codes of the G query heads (the exact count, which the scan never forms).
template <int G>
__global__ __launch_bounds__(256) void counts_kernel(DecodeArgs a)
{
    const int gc = blockIdx.x;
    const int bkv = gc / a.n_chunks, chunk = gc - bkv * a.n_chunks;
    const int bhq0 = (bkv / a.H_kv) * a.H_q + (bkv % a.H_kv) * G;
    const int t = threadIdx.x, kw = t >> 4, ksh = 2 * (t & 15);
    const int n = a.n, K = a.K, Kr = a.Kr;
    const uint32_t *pc = a.planes + (int64_t(bkv) * a.nc_cap + chunk) * a.L * Kr * kWords + kw;
    uint32_t cnt[2][G] = {};
    for (int l = 0; l < a.L; ++l) {
        uint32_t code0 = 0u, code1 = 0u;
        for (int b = 0; b < K; ++b) {
            const uint32_t wv = pc[(int64_t(l) * Kr + b) * kWords] >> ksh;
            code0 |= (wv & 1u) << b;
            code1 |= ((wv >> 1) & 1u) << b;
        }
        for (int g = 0; g < G; ++g) {
            const uint32_t qc = a.qcodes[int64_t(bhq0 + g) * a.L + l];
            cnt[0][g] += code0 == qc;
            cnt[1][g] += code1 == qc;
        }
    }
    const int64_t key0 = int64_t(chunk) * kChunk + 2 * t;
    for (int e = 0; e < 2; ++e)
        if (key0 + e < n)
            for (int g = 0; g < G; ++g)
                a.counts[int64_t(bhq0 + g) * n + key0 + e] = uint8_t(cnt[e][g]);
}

// ---------------------------------------------------------------- merge
// Block = one (KV head unit, query head g of its group, kMergeDims dims);
// thread = (dim c of kMergeDims, record lane j of 32).  A unit's records are
// its runs of `cpb` chunks (cpb = 1: one record a chunk): the unit's chunks
// [u n_chunks, (u+1) n_chunks) meet runs floor(u n_chunks / cpb) through
// floor(((u+1) n_chunks - 1) / cpb).  Lane j folds records j, j+32, ... into
// a running (max, sum, acc), loading NB records before folding them so their
// loads overlap; NB is the smallest of 1, 2, 3, 4, 6, 8 that covers a unit's
// records in one pass (loads past the last record are wasted: 8 a lane at
// 64 records took the 96K step 0.7 us longer than 2).  The 32 lanes are then
// combined by a fixed tree (lanes j and j + 16, then j and j + 8, ...), so
// the result is deterministic.  16 dims a block (256 blocks at 32 query
// heads) spread the launch over the CUs.
constexpr int kMergeDims = 16;
template <int G, int NB>
__global__ __launch_bounds__(32 * kMergeDims) void merge_kernel(const float *__restrict__ part,
                                                    int32_t n_chunks, int32_t cpb, int32_t H_kv,
                                                    int32_t H_q, float *__restrict__ out)
{
    __shared__ float sm[32][kMergeDims + 1], sl[32][kMergeDims + 1], sa[32][kMergeDims + 1];
    const int bkv = blockIdx.x / G, g = blockIdx.x % G;
    const int t = threadIdx.x, cl = t % kMergeDims, j = t / kMergeDims;
    const int c = kMergeDims * blockIdx.y + cl;
    const int64_t first = int64_t(bkv) * n_chunks;
    const int nrec = int((first + n_chunks - 1) / cpb - first / cpb + 1);
    const float *p = part + first * (G * kPart) + g * kPart;
    float m = -INFINITY, l = 0.0f, acc = 0.0f;
    for (int base = j; base < nrec; base += 32 * NB) {
        float mb[NB], lb[NB], ab[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int ch = base + 32 * u;
            const float *pc = p + int64_t(min(ch, nrec - 1)) * (G * kPart);
            mb[u] = pc[0];
            lb[u] = pc[1];
            ab[u] = pc[2 + c];
            if (ch >= nrec) mb[u] = -INFINITY;   // past the last record: nothing
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const float mc = mb[u], lc = lb[u], ac = ab[u];
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
    }
    sm[j][cl] = m;
    sl[j][cl] = l;
    sa[j][cl] = acc;
    for (int half = 16; half >= 1; half >>= 1) {
        __syncthreads();
        if (j < half) {
            const float m2 = sm[j + half][cl], l2 = sl[j + half][cl], a2 = sa[j + half][cl];
            const float M = fmaxf(m, m2);
            if (M != -INFINITY) {   // both empty: nothing
                const float f1 = __expf(m - M), f2 = __expf(m2 - M);
                l = fmaf(l, f1, l2 * f2);
                acc = fmaf(acc, f1, a2 * f2);
                m = M;
            }
            sm[j][cl] = m;
            sl[j][cl] = l;
            sa[j][cl] = acc;
        }
    }
    if (j == 0) {
        const int b = bkv / H_kv, h = bkv % H_kv;
        out[(int64_t(b) * H_q + h * G + g) * kD + c] = l > 0.0f ? acc / l : 0.0f;
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

// Workgroups the grid of scan_gather_kernel<G, T, KP> is sized for on the
// current device: compute units x workgroups resident per unit, but at most
// two per unit up to G = 4, cached per device.  Two with longer runs finish
// sooner there than three: the oldest-first wave scheduler leaves the third
// workgroup of a unit to run its last chunk nearly alone.  With G = 8 the
// gather's arithmetic needs the third workgroup's waves.
template <int G, typename T, int KP>
int resident_workgroups()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_gather_kernel<G, T, KP>, 256,
                                                         0) != hipSuccess)
            return 0;
        if (G <= 4 && per_cu > 2) per_cu = 2;
        cached[dev] = cus * (per_cu > 0 ? per_cu : 1);
    }
    return cached[dev];
}

template <int G, typename T, int KP>
hipError_t launch_scan_gather_t(const DecodeArgs &a, hipStream_t s, int32_t &cpb)
{
    const int64_t chunks = int64_t(a.B) * a.H_kv * a.n_chunks;
    const int slots = resident_workgroups<G, T, KP>();
    if (slots <= 0) return hipErrorInvalidDevice;
    cpb = ceil_div(chunks, slots);
    const dim3 grid(ceil_div(chunks, cpb));
    // timed entry point: the runtime stamps the events at this kernel's own
    // start and end
    return launch_timed(scan_gather_kernel<G, T, KP>, grid, dim3(256), 0, s, a.ev_begin, a.ev_end,
                        a, cpb, fused_merge_records(a, G, cpb, kFusedMergeMax));
}

template <int G, typename T>
hipError_t launch_scan_gather_kp(const DecodeArgs &a, hipStream_t s, int32_t &cpb)
{
    switch (plane_rows_class(a.Kr)) {
    case 4: return launch_scan_gather_t<G, T, 4>(a, s, cpb);
    case 8: return launch_scan_gather_t<G, T, 8>(a, s, cpb);
    case 9: return launch_scan_gather_t<G, T, 9>(a, s, cpb);
    case 10: return launch_scan_gather_t<G, T, 10>(a, s, cpb);
    case 12: return launch_scan_gather_t<G, T, 12>(a, s, cpb);
    default: return launch_scan_gather_t<G, T, 16>(a, s, cpb);
    }
}

// Launches scan_gather; cpb receives its run length (chunks a workgroup).
template <int G>
hipError_t launch_scan_gather(const DecodeArgs &a, hipStream_t s, int32_t &cpb)
{
    return a.dtype == MP_BF16 ? launch_scan_gather_kp<G, uint16_t>(a, s, cpb)
                              : launch_scan_gather_kp<G, float>(a, s, cpb);
}

}  // namespace

// ---- launches shared with the bucketed-table path (tables.hip) ----
namespace {
template <int QH, typename T>
hipError_t launch_encode_append_t(const DecodeArgs &a, hipStream_t s)
{
    const int BHq = a.B * a.H_q;
    const int TB = a.K > 0 ? 64 / a.K : 64;
    const int nbx = ceil_div(a.L, TB), nby = ceil_div(BHq, QH), n_enc = encode_grid(nbx, nby);
    const int nhb = ceil_div(int64_t(a.K) * a.L, kAppendRows);
    const int units = a.B * a.H_kv;
    return launch(encode_append_kernel<QH, T>, dim3(n_enc + units * nhb), dim3(256), 0, s, a.q, BHq,
                  a.W, a.K, a.L, a.qcodes, a.qq, a.qnorm, nbx, nby, n_enc,
                  static_cast<const T *>(a.k.data), a.k.sb, a.k.sh, a.k.sn, a.H_kv, a.app_n0, a.n,
                  a.nc_cap, a.mu, a.app_planes, nhb, a.unit_cnt, a.unit_cnt ? units : 0);
}

// The query encode with the append of keys [app_n0, n) (1 to kAppendMax, K > 0).
hipError_t launch_encode_append(const DecodeArgs &a, hipStream_t s)
{
    if (a.n - a.app_n0 < 1 || a.n - a.app_n0 > kAppendMax || a.K <= 0 || !a.app_planes)
        return hipErrorInvalidValue;
    const bool small = a.B * a.H_q <= 32;
    if (a.dtype == MP_BF16)
        return small ? launch_encode_append_t<2, uint16_t>(a, s)
                     : launch_encode_append_t<4, uint16_t>(a, s);
    return small ? launch_encode_append_t<2, float>(a, s) : launch_encode_append_t<4, float>(a, s);
}
}  // namespace

hipError_t launch_encode_query(const DecodeArgs &a, hipStream_t s)
{
    const int BHq = a.B * a.H_q;
    const int TB = a.K > 0 ? 64 / a.K : 64;
    const int nbx = ceil_div(a.L, TB);
    const int ncnt = a.unit_cnt ? a.B * a.H_kv : 0;
    if (BHq <= 32) {
        const int nby = ceil_div(BHq, 2);
        return launch(encode_query_kernel<2>, dim3(encode_grid(nbx, nby)), dim3(256), 0, s, a.q,
                      BHq, a.W, a.K, a.L, a.qcodes, a.qq, a.qnorm, nbx, nby, a.unit_cnt, ncnt);
    }
    const int nby = ceil_div(BHq, 4);
    return launch(encode_query_kernel<4>, dim3(encode_grid(nbx, nby)), dim3(256), 0, s, a.q, BHq,
                  a.W, a.K, a.L, a.qcodes, a.qq, a.qnorm, nbx, nby, a.unit_cnt, ncnt);
}

namespace {
// The merge with NB records a lane per load batch: the smallest of 1, 2, 3,
// 4, 6, 8 whose 32 NB slots hold a unit's records (n_chunks / cpb where runs
// align with units, else at most ceil(n_chunks / cpb) + 1).
template <int G>
hipError_t launch_merge_g(const DecodeArgs &a, int32_t cpb, hipStream_t s)
{
    const dim3 grid(a.B * a.H_kv * G, kD / kMergeDims), block(32 * kMergeDims);
    const float *part = a.part;
    const int32_t nc = a.n_chunks;
    const int64_t nrec = nc % cpb == 0 ? nc / cpb : (int64_t(nc) + cpb - 1) / cpb + 1;
    if (nrec <= 32)
        return launch(merge_kernel<G, 1>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
    if (nrec <= 64)
        return launch(merge_kernel<G, 2>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
    if (nrec <= 96)
        return launch(merge_kernel<G, 3>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
    if (nrec <= 128)
        return launch(merge_kernel<G, 4>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
    if (nrec <= 192)
        return launch(merge_kernel<G, 6>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
    return launch(merge_kernel<G, 8>, grid, block, 0, s, part, nc, cpb, a.H_kv, a.H_q, a.out);
}
}  // namespace

hipError_t launch_merge(const DecodeArgs &a, int32_t cpb, hipStream_t s)
{
    switch (a.G) {
    case 1: return launch_merge_g<1>(a, cpb, s);
    case 2: return launch_merge_g<2>(a, cpb, s);
    case 4: return launch_merge_g<4>(a, cpb, s);
    case 8: return launch_merge_g<8>(a, cpb, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_counts(const DecodeArgs &a, hipStream_t s)
{
    if (!a.debug || !a.counts) return hipSuccess;
    const dim3 grid(a.B * a.H_kv * a.n_chunks);
    switch (a.G) {
    case 1: return launch(counts_kernel<1>, grid, dim3(256), 0, s, a);
    case 2: return launch(counts_kernel<2>, grid, dim3(256), 0, s, a);
    case 4: return launch(counts_kernel<4>, grid, dim3(256), 0, s, a);
    case 8: return launch(counts_kernel<8>, grid, dim3(256), 0, s, a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_seg_compact(const DecodeArgs &a, hipStream_t s)
{
    if (!a.debug || (!a.s_idx && !a.s_len)) return hipSuccess;
    return launch(seg_compact_kernel, dim3(a.B * a.H_q), dim3(256), 0, s, a.seg_idx, a.seg_cnt,
                  a.n_chunks, a.n, a.s_idx, a.s_len);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    // a decode that first appends keys [app_n0, n) writes their codes in the
    // query encode's launch
    hipError_t e = a.app_n0 < a.n ? launch_encode_append(a, s) : launch_encode_query(a, s);
    if (e != hipSuccess) return e;
    int32_t cpb = 1;
    switch (a.G) {
    case 1: e = launch_scan_gather<1>(a, s, cpb); break;
    case 2: e = launch_scan_gather<2>(a, s, cpb); break;
    case 4: e = launch_scan_gather<4>(a, s, cpb); break;
    case 8: e = launch_scan_gather<8>(a, s, cpb); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // the merge runs inside scan_gather where runs align with units
    if (fused_merge_records(a, a.G, cpb, kFusedMergeMax) == 0 &&
        (e = launch_merge(a, cpb, s)) != hipSuccess)
        return e;
    if ((e = launch_counts(a, s)) != hipSuccess) return e;
    return launch_seg_compact(a, s);
}

}  // namespace mp
