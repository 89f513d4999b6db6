/*
 * magicpig.h -- C ABI of the MI355X (gfx950) MagicPIG decode-attention library.
 *
 * What it computes.  MagicPIG estimates one decode step of softmax attention
 * by locality-sensitive-hash sampling:
 *   - keys are centered by their mean and SimHash-encoded into L tables of K
 *     sign bits each (page "MagicPIG: LSH Sampling for Efficient LLM
 *     Generation", method details: the K x L random projections and the
 *     centering step; page "MagicPIG: don't pick the tallest", section 5);
 *   - a query samples every key that shares its bucket in at least two tables;
 *   - each sampled key i is weighted by exp(q.k_i/sqrt(d) - log u_i), where
 *     u_i = 1 - (1-p_i^K)^L - L p_i^K (1-p_i^K)^(L-1) and
 *     p_i = 1 - arccos(cos(q, k_i - mu))/pi (the summary page's quick-read
 *     equations and its algorithm steps);
 *   - the sink and local tokens T are attended exactly (u = 1), and one
 *     softmax over [sampled, exact] gives the output (system co-design
 *     section: on-device cache of sink/local tokens merged with the sampled
 *     part).
 * The two calls follow the pages' problem statement (background section):
 * build the index once per key cache, then estimate o = softmax(qK^T/sqrt d)V
 * from a sampled subset per decode step.
 *
 * Conventions for every call:
 *   - every tensor pointer is a DEVICE pointer (HBM of the current HIP device);
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream); all
 *     work is enqueued on it asynchronously and nothing here synchronises;
 *   - the library never allocates device memory: the caller owns keys, values,
 *     queries, outputs, the index workspace and the decode scratch;
 *   - arguments are validated on the host before anything is enqueued; on any
 *     status other than MP_OK nothing has been enqueued (except MP_E_HIP, which
 *     reports that one of the call's own launches failed: launches before it
 *     in the same call stay enqueued), and mp_last_error() describes the
 *     problem.  MP_E_HIP comes from the status each launch returns, never from
 *     an error an earlier, unrelated HIP call left behind;
 *   - index handles are checked against the library's list of live handles
 *     before use: a destroyed handle gives MP_E_HANDLE, not a read of freed
 *     memory;
 *   - device faults surface at the caller's next synchronisation of the stream;
 *   - head dimension d must be 128.
 *
 * Fixed readings (where the pages leave a choice open):
 *   - hyperplanes: W is [R][128] fp32 row-major, R = K*L, row j = l*K + b is
 *     bit b of table l.  Element e = j*128 + c is the Box-Muller standard normal
 *     sqrt(-2 ln u1) cos(2 pi u2) (computed in fp64, rounded to fp32) of
 *     u1 = ((z1 >> 11) + 1) 2^-53 and u2 = (z2 >> 11) 2^-53, where z1, z2 are
 *     the outputs number 2e+1 and 2e+2 of SplitMix64 (Steele, Lea & Flood 2014)
 *     started at `seed`.  A smaller L therefore uses a row prefix of W.
 *   - sign bit = 1 iff projection > 0; code of table l packs bit b at 2^b.
 *   - queries are hashed raw; keys are hashed after subtracting the mean of
 *     all n keys of their (sequence, KV head), sink and local tokens included.
 *   - the cosine in p_i uses the centered key; scores use the raw key.
 *   - T = [0, n_sink) u [n - n_local, n); sampled sets exclude T.
 *   - query head h of a sequence uses KV head h / G, G = H_q / H_kv.
 *   - a zero-length query or centered key has cosine 0.
 */
#ifndef MAGICPIG_H
#define MAGICPIG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mp_status {
    MP_OK = 0,
    MP_E_ARG = 1,        /* null pointer, value out of range */
    MP_E_SHAPE = 2,      /* shapes/strides disagree or are unsupported */
    MP_E_DTYPE = 3,      /* unsupported dtype */
    MP_E_WORKSPACE = 4,  /* workspace/scratch too small or misaligned */
    MP_E_HIP = 5,        /* a HIP call or kernel launch failed */
    MP_E_HANDLE = 6      /* index handle is NULL or not a live index */
} mp_status;

typedef enum mp_dtype { MP_F32 = 0, MP_BF16 = 1 } mp_dtype;

/* A [B][H][n][d] key or value tensor.  Strides are in elements; the d axis is
 * contiguous.  `data` and every row start must be 16-byte aligned. */
typedef struct mp_kv_view {
    const void *data;
    int32_t dtype;               /* mp_dtype */
    int32_t B, H, n, d;
    int64_t stride_b, stride_h, stride_n;
} mp_kv_view;

/* Opaque host handle of a built index; it points into the caller's workspace. */
typedef struct mp_index mp_index;

/* Keys per chunk of the code layout (see mp_index_views). */
#define MP_CHUNK 512

/* Most keys per (sequence, KV head) an index or a view may hold (2^30: key
 * counts padded to whole chunks stay inside int32).  Views with more keys are
 * MP_E_SHAPE; size queries for more return 0. */
#define MP_MAX_KEYS (1 << 30)

/* Bytes of device workspace mp_build_index needs for these sizes; 0 if the
 * sizes are invalid (B, H_kv >= 1, B * H_kv <= 65535; 1 <= n <= MP_MAX_KEYS;
 * d == 128; 0 <= K <= 16; 2 <= L <= 255). */
size_t mp_index_workspace_bytes(int32_t B, int32_t H_kv, int32_t n, int32_t d,
                                int32_t K, int32_t L);

/* Build the index of `keys` ([B][H_kv][n][128], fp32 or bf16): hyperplanes W
 * from `seed`, per-(sequence, KV head) mean mu, and the codes of every key
 * (K bits per key and table, stored as bit planes: see mp_index_views).
 * The index holds W, mu and the codes only; keys and values are not copied,
 * and decode reads them again through its own views.  The workspace
 * (>= mp_index_workspace_bytes, 256-byte aligned) must stay alive and
 * unmodified while the index is used.  *out receives a host handle (free it
 * with mp_index_destroy).  Ownership of `keys` stays with the caller; the
 * keys must not change until the enqueued build has run. */
mp_status mp_build_index(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                         void *workspace, size_t workspace_bytes, void *stream,
                         mp_index **out);

/* Build flags of mp_build_index_ex.
 * MP_INDEX_MIPS: the inner-product-to-cosine lift of page "MagicPIG: LSH
 *   Sampling for Efficient LLM Generation", method details (variance
 *   reduction with LSH): with x_i = k_i - mu the centered key and
 *   r = max_i |x_i|, each key is hashed as [x_i, sqrt(r^2 - |x_i|^2)] and the
 *   query as [q, 0], against hyperplanes [W_j, w_j] whose extra coordinate
 *   w_j is normal number K*L*128 + j of the hyperplane stream; p_i then uses
 *   the lifted cosine q.x_i / (|q| r).  |x_i|^2 and r^2 are formed in fp64.
 *   Such an index cannot grow (r would move): mp_index_append refuses it. */
#define MP_INDEX_MIPS 1

/* Workspace bytes of an index built with `flags` (mp_index_workspace_bytes
 * is flags = 0); 0 if invalid. */
size_t mp_index_workspace_bytes_ex(int32_t B, int32_t H_kv, int32_t n, int32_t d, int32_t K,
                                   int32_t L, int32_t flags);

/* mp_build_index_cap with build flags (MP_INDEX_*); the workspace must hold
 * mp_index_workspace_bytes_ex(B, H_kv, n_cap, 128, K, L, flags) bytes.
 * MP_E_ARG for unknown flags. */
mp_status mp_build_index_ex(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                            int32_t n_cap, int32_t flags, void *workspace,
                            size_t workspace_bytes, void *stream, mp_index **out);

/* Device pointers to the lift of an MP_INDEX_MIPS index: w_extra [K*L] fp32
 * (the hyperplanes' extra coordinate), r [B][H_kv] fp32 (the lift radius of
 * each unit).  MP_E_ARG for an index built without the lift. */
mp_status mp_index_lift_views(const mp_index *idx, const float **w_extra, const float **r);

/* mp_build_index over the n keys of `keys` into an index that
 * mp_index_append can later grow to n_cap keys (n <= n_cap): the workspace
 * must hold mp_index_workspace_bytes(B, H_kv, n_cap, 128, K, L) bytes.
 * MP_E_ARG if n_cap < n or n_cap is not a valid key count. */
mp_status mp_build_index_cap(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                             int32_t n_cap, void *workspace, size_t workspace_bytes,
                             void *stream, mp_index **out);

/* Grow an index to the first keys->n keys of its key cache: the keys past the
 * index's n are centered by the mean mu fixed at build time and encoded with
 * the index's hyperplanes, so a token that leaves the exact local window can
 * join the sampled keys without a rebuild (page "MagicPIG: LSH Sampling for
 * Efficient LLM Generation", system co-design: the sink and local tokens sit
 * in a static cache beside the hashed keys; the pages do not say how mu
 * moves as keys arrive: here it stays as built).
 *   keys   the index's key cache viewed with its new length: [B][H_kv][n_new][128],
 *          same B, H_kv and dtype, index's n <= n_new <= n_cap; its first n
 *          keys must be the ones indexed.
 * The enqueued encode also rewrites the plane words of the last 256 keys
 * already indexed, with the same bits; decodes that read the index on other
 * streams must be ordered with it.  The index then covers n_new keys: decode
 * calls must pass K/V views of that length.  Bucketed tables built before are
 * detached (the table calls then return MP_E_ARG until mp_build_tables runs
 * again with a workspace for the new n).
 * MP_E_HANDLE for a dead handle, MP_E_DTYPE / MP_E_SHAPE for keys that do not
 * fit, MP_E_ARG when called on another device than the index's or for an
 * index built with MP_INDEX_MIPS. */
mp_status mp_index_append(mp_index *idx, const mp_kv_view *keys, void *stream);

/* Bytes of device scratch one mp_decode_attn / mp_decode_debug /
 * mp_decode_attn_append call needs for H_q query heads per sequence, for the
 * index grown to its capacity n_cap (so one scratch serves every call as the
 * index grows; n_cap = n for an index built without room); 0 if invalid. */
size_t mp_decode_scratch_bytes(const mp_index *idx, int32_t H_q);

/* One decode step for every (sequence, query head).
 *   q      [B][H_q][128] fp32, contiguous; H_q = G * H_kv with G in {1,2,4,8}
 *   k, v   the key and value caches the index was built from: [B][H_kv][n][128],
 *          same dtype (fp32 or bf16)
 *   n_sink, n_local >= 0   the exact set T
 *   scale  score scale; 0 means 1/sqrt(128)
 *   out    [B][H_q][128] fp32, contiguous
 *   scratch >= mp_decode_scratch_bytes(idx, H_q), 256-byte aligned; calls that
 *          share one scratch buffer must be ordered on one stream.
 * Several decodes may read one index concurrently. */
mp_status mp_decode_attn(const float *q, int32_t H_q, const mp_index *idx,
                         const mp_kv_view *k, const mp_kv_view *v,
                         int32_t n_sink, int32_t n_local, float scale, float *out,
                         void *scratch, size_t scratch_bytes, void *stream);

/* mp_index_append(idx, k, stream) followed by mp_decode_attn over the grown
 * index, with the new keys' codes written by the decode's first launch: one
 * kernel launch fewer a step for a decode that appends the token leaving the
 * exact local window (page "MagicPIG: LSH Sampling for Efficient LLM
 * Generation", system co-design: the sink and local tokens sit in a static
 * cache beside the hashed keys).
 *   k, v   the key and value caches viewed with the new length n_new:
 *          [B][H_kv][n_new][128]; index's n <= n_new <= n_cap, and the first
 *          n keys of k must be the ones indexed
 *   other arguments as mp_decode_attn; scratch >= mp_decode_scratch_bytes.
 * 1 to 64 new keys ride on the decode's query-encode launch; more keys, or
 * K = 0, take mp_index_append and then mp_decode_attn.  Either way the
 * results are bit-identical to the two calls.  Every argument is checked
 * before anything is enqueued: a refused call (MP_E_HANDLE, MP_E_ARG for a
 * lifted index or another device, MP_E_DTYPE, MP_E_SHAPE, MP_E_WORKSPACE)
 * leaves the index unchanged.  MP_E_HIP (a failed launch) may leave the new
 * keys' bits in plane words past n, which no decode reads, or, on the
 * two-call route, the index grown.  Like mp_index_append it changes the index
 * (n, detached tables): no other call on the index may overlap it. */
mp_status mp_decode_attn_append(const float *q, int32_t H_q, mp_index *idx,
                                const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                int32_t n_local, float scale, float *out, void *scratch,
                                size_t scratch_bytes, void *stream);

/* Bytes of the static device array behind mp_decode_attn_noalloc. */
#define MP_NOALLOC_SCRATCH_BYTES (32u << 20)

/* mp_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * It takes no scratch argument: its scratch is a static device array of the
 * library, MP_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU it runs on, held
 * from the library's load until the process ends; the call itself allocates
 * nothing.  Arguments, layouts and the output are those of mp_decode_attn
 * (the same kernels, bit-identical results).  The scratch it needs, 256-byte
 * aligned pieces of B*H_q*L*2 + B*H_q*L*4 + B*H_q*4 + B*H_q*ceil(n/512)*130*4
 * + B*H_kv*4 bytes (query codes, their packed form, norms, partial records,
 * per-unit record counts), must fit the array: MP_E_WORKSPACE otherwise,
 * before anything is enqueued.  All calls on
 * one GPU share that GPU's array, so calls that overlap on one GPU (other
 * streams or threads) race; order them on one stream. */
mp_status mp_decode_attn_noalloc(const float *q, int32_t H_q, const mp_index *idx,
                                 const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                 int32_t n_local, float scale, float *out, void *stream);

/* mp_decode_attn plus the intermediate results, each optional (NULL = skip):
 *   qcodes [B][H_q][L] uint16     query codes
 *   counts [B][H_q][n] uint8      tables in which key i shares the query's bucket
 *   s_idx  [B][H_q][n] int32      sampled set S (ascending; T excluded), padded
 *   s_len  [B][H_q]    int32      |S|
 * The output equals what mp_decode_attn computes. */
mp_status mp_decode_debug(const float *q, int32_t H_q, const mp_index *idx,
                          const mp_kv_view *k, const mp_kv_view *v,
                          int32_t n_sink, int32_t n_local, float scale, float *out,
                          void *scratch, size_t scratch_bytes, void *stream,
                          uint16_t *qcodes, uint8_t *counts, int32_t *s_idx, int32_t *s_len);

/* ---- Bucketed hash tables (the retrieval of the summary page's algorithm
 * steps: the query's code selects one bucket per table, and the keys found in
 * at least two buckets are sampled; page "MagicPIG: don't pick the tallest",
 * section 6: one 32-bit token index per key and table).  They give the same
 * sampled sets and outputs as mp_decode_attn, reading the query's L buckets
 * instead of every key's codes.  Supported for K <= 12 and
 * ceil(n/512)*128 + 4*(2L + 1) <= 162,816 bytes (a head's 2-bit-per-key
 * collision bitmap and its bucket bounds in one workgroup's LDS), which holds
 * for every L up to n = 643,072. ---- */

/* Bytes of the table workspace of an index (256-byte aligned):
 *   offsets [B*H_kv][L][2^K + 1] uint32: bucket b of table l of unit u holds
 *           entries [offsets[u][l][b], offsets[u][l][b+1]) of that table;
 *   entries [B*H_kv][L][n] uint32: key indices grouped by bucket (their order
 *           within a bucket is not fixed; nothing depends on it).
 * 0 if the index cannot have tables (K > 12, n too large, not a live index). */
size_t mp_tables_workspace_bytes(const mp_index *idx);

/* Builds the tables of `idx` from its codes into `workspace` (caller-owned,
 * at least mp_tables_workspace_bytes, 256-byte aligned, kept alive and
 * unchanged while the index is used with the calls below) and attaches them
 * to the index.  A later call rebuilds them into the new workspace.
 * MP_E_SHAPE if the index cannot have tables. */
mp_status mp_build_tables(mp_index *idx, void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes of mp_decode_attn_tables / _timed / _debug for H_q query
 * heads (0 if invalid).  Larger than mp_decode_scratch_bytes by the per-head
 * collision bitmaps, 2 bits per key. */
size_t mp_decode_tables_scratch_bytes(const mp_index *idx, int32_t H_q);

/* mp_decode_attn through the tables built by mp_build_tables (MP_E_ARG if
 * none); arguments, layouts and errors as for mp_decode_attn. */
mp_status mp_decode_attn_tables(const float *q, int32_t H_q, const mp_index *idx,
                                const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                int32_t n_local, float scale, float *out, void *scratch,
                                size_t scratch_bytes, void *stream);

/* mp_decode_tables with the debug views of mp_decode_debug, except that
 * counts2[b][h][i] = min(collision count, 2): the tables only tell whether a
 * key was seen once or at least twice. */
mp_status mp_decode_tables_debug(const float *q, int32_t H_q, const mp_index *idx,
                                 const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                 int32_t n_local, float scale, float *out, void *scratch,
                                 size_t scratch_bytes, void *stream, uint16_t *qcodes,
                                 uint8_t *counts2, int32_t *s_idx, int32_t *s_len);

/* Device pointers to the attached tables (layout above); MP_E_ARG if none. */
mp_status mp_tables_views(const mp_index *idx, const uint32_t **offsets, const uint32_t **entries);

/* Device pointers into the index workspace (valid while the workspace is):
 *   W      [R][128] fp32, R = K*L
 *   mu     [B][H_kv][128] fp32
 *   planes the key codes as bit planes, [B][H_kv][nc][L*Kr][MP_CHUNK/32]
 *          uint32 with Kr = max(K, 1) and nc = ceil(n_cap / MP_CHUNK) chunks
 *          per (sequence, KV head) (n_cap = n unless built by
 *          mp_build_index_cap); *n_pad/MP_CHUNK of them hold keys: bit j of
 *          word w of row l*Kr + b of chunk c is bit b of the table-l code of
 *          key c*MP_CHUNK + 32*w + j (K bits per key and table, the code's
 *          own width).  With K = 0 every code is 0 and the one row per table
 *          is zero.  Keys i >= n are padding and never sampled.
 * Any output pointer may be NULL. */
mp_status mp_index_views(const mp_index *idx, const float **W, const float **mu,
                         const uint32_t **planes, int32_t *n_pad);

/* Free the host handle (not the workspace).  NULL and handles that are not
 * live are ignored. */
void mp_index_destroy(mp_index *idx);

/* Static description of a status code. */
const char *mp_status_str(mp_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *mp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MAGICPIG_H */
