// mp_internal.h -- types and launchers shared by the HIP sources of libmagicpig.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <tuple>
#include <utility>

#include "../../include/magicpig.h"
#include "../../include/magicpig_bench.h"
#include "../../include/magicpig_testing.h"

namespace mp {

constexpr int kD = 128;            // head dimension
constexpr int kChunk = MP_CHUNK;   // keys per scan chunk: 64 lanes x 8 keys
constexpr int kWords = kChunk / 32;   // 32-key words per chunk and plane row
constexpr int kMeanRows = 1024;    // keys per partial-sum block of the mean pass

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
inline int32_t ceil_div(int64_t a, int64_t b) { return int32_t((a + b - 1) / b); }

// ---- kernel launches that report their own status ----
// Launches fail on request of mp_debug_fail_launches (a test aid): the next
// `skip` launches run, then each of the following `count` launches returns
// hipErrorLaunchFailure without launching.  Both counts live in one word
// (skip << 32 | count) so that concurrent launches take them consistently.
extern std::atomic<uint64_t> g_forced_launch_failures;
inline bool take_forced_failure()
{
    uint64_t v = g_forced_launch_failures.load(std::memory_order_relaxed);
    for (;;) {
        if (v == 0) return false;
        const uint64_t skip = v >> 32, count = v & 0xFFFFFFFFu;
        const uint64_t next = skip > 0 ? ((skip - 1) << 32 | count) : (count - 1);
        if (g_forced_launch_failures.compare_exchange_weak(v, next, std::memory_order_relaxed))
            return skip == 0;
    }
}

template <typename... P, size_t... I>
hipError_t launch_packed(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         hipEvent_t ev0, hipEvent_t ev1, std::tuple<P...> &args,
                         std::index_sequence<I...>)
{
    void *argv[sizeof...(P) + 1] = {static_cast<void *>(&std::get<I>(args))..., nullptr};
    if (take_forced_failure()) return hipErrorLaunchFailure;
    if (ev0 || ev1)
        return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, s,
                                  ev0, ev1, 0);
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, s);
}

// kernel<<<grid, block, lds, s>>>(args...), returning the status of this
// launch (hipLaunchKernel), not an error left behind by an earlier call.
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  A &&...args)
{
    std::tuple<P...> t(std::forward<A>(args)...);
    return launch_packed(kernel, grid, block, lds, s, nullptr, nullptr, t,
                         std::index_sequence_for<P...>{});
}

// The same, with two events the runtime stamps at the kernel's own start and
// end (hipExtLaunchKernel); both NULL is a plain launch.
template <typename... P, typename... A>
hipError_t launch_timed(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                        hipEvent_t ev0, hipEvent_t ev1, A &&...args)
{
    std::tuple<P...> t(std::forward<A>(args)...);
    return launch_packed(kernel, grid, block, lds, s, ev0, ev1, t,
                         std::index_sequence_for<P...>{});
}

// Runs a set-up step (a kernel attribute, a symbol lookup) once per device:
// the first call on the current device runs f(), later calls return hipSuccess
// once it has succeeded (a failed step is tried again next time).
class PerDevice {
  public:
    template <typename F> hipError_t once(F f)
    {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (done_[dev].load(std::memory_order_acquire)) return hipSuccess;
        std::lock_guard<std::mutex> g(m_);
        if (done_[dev].load(std::memory_order_relaxed)) return hipSuccess;
        e = f(dev);
        if (e == hipSuccess) done_[dev].store(true, std::memory_order_release);
        return e;
    }
    static constexpr int kMaxDevices = 64;

  private:
    std::mutex m_;
    std::atomic<bool> done_[kMaxDevices] = {};
};

// Workspace layout of an index (all offsets 256-byte aligned).
struct IndexLayout {
    int32_t B, H_kv, n, n_pad, n_chunks, n_mean_blocks, K, L, R, R_pad;
    int32_t Kr;        // plane rows per table: K, or 1 (all zero) when K = 0
    int32_t n_cap, nc_cap;   // keys the index may grow to; plane chunks per unit
    int32_t flags;           // MP_INDEX_* of the build
    int64_t off_W, off_Wp, off_mu, off_mu_part, off_planes, total;
    // inner-product-to-cosine lift (MP_INDEX_MIPS only; 0 otherwise)
    int64_t off_wx, off_mu64, off_xx, off_xmax, off_r2, off_rn;
};
// Layout of an index over n keys with room for n_cap >= n (regions sized for
// n_cap; the n-dependent counts describe the n keys).
IndexLayout index_layout(int32_t B, int32_t H_kv, int32_t n, int32_t K, int32_t L,
                         int32_t n_cap = 0, int32_t flags = 0);

struct mp_index_impl {
    IndexLayout lay;
    uint64_t seed;
    int32_t key_dtype;
    int device;
    float *W;        // [R_pad][128] canonical (rows >= R are zero)
    float *Wp;       // [R_pad/16][8][64][4] MFMA B-fragment order
    float *mu;       // [B*H_kv][128]
    double *mu_part; // [B*H_kv][n_mean_blocks][128]
    uint32_t *planes; // [B*H_kv][n_chunks][L*Kr][kWords]: bit j of word w of row
                      // l*Kr + b is bit b of the code of key 32w + j in table l
    // inner-product-to-cosine lift (NULL unless built with MP_INDEX_MIPS)
    float *wx;       // [R_pad] lifted coordinate of each hyperplane
    double *mu64;    // [B*H_kv][128] mean in fp64
    double *xx;      // [B*H_kv][n_cap] |k_i - mu|^2 in fp64
    double *xmax;    // [B*H_kv][n_mean_blocks] per-block max of xx
    double *r2;      // [B*H_kv] r^2 = max_i xx_i
    float *rnorm;    // [B*H_kv] r
    // bucketed tables, once built (NULL until then)
    uint32_t *tab_off; // [B*H_kv][L][2^K + 1] bucket starts
    uint32_t *tab_ent; // [B*H_kv][L][n] keys, grouped by bucket
};

// Workspace layout of the bucketed tables of an index.
constexpr int kMaxTableK = 12;   // 2^K bucket counters live in LDS while a table is built
// Largest dynamic LDS of the bucket walk (a head's collision bitmap and its
// bucket bounds): a workgroup's 160 KB less room for the static part.
constexpr size_t kCollideLdsMax = 160 * 1024 - 1024;
// The bucket walk of the table path: `slices` workgroups per query head, each
// over L / slices of its tables, and whether they compute the query's codes
// for their tables themselves (one launch fewer, at the price of reading W
// once per query head instead of once per four).  Both depend only on the
// number of query heads B * H_q, so the scratch layout and the launch agree.
// The gather is compiled for 4 and 8 slices.
constexpr int kMaxCollideSlices = 8;
struct CollidePlan {
    int32_t slices;
    bool own_codes;
};
inline CollidePlan collide_plan(int64_t BHq)
{
    if (BHq <= 32) return {8, true};
    if (BHq <= 64) return {4, true};
    return {4, false};
}
// Dynamic LDS of the bucket walk of an index: 2 bits per key, 2L + 1 bucket words.
size_t collide_lds_bytes(const IndexLayout &lay);
struct TablesLayout {
    int32_t nbins;
    int64_t off_offsets, off_entries, total;
};
TablesLayout tables_layout(const IndexLayout &lay);

// Decode scratch layout.
struct DecodeLayout {
    int32_t BHq, n_chunks;
    int64_t off_qcodes, off_qq, off_qnorm, off_part, off_cnt, off_seg_idx, off_seg_cnt, off_bits,
        total;
};
// `tables`: also the per-head collision bitmaps of the bucketed-table path;
// `debug`: also the per-chunk sampled lists of the debug entry points.
DecodeLayout decode_layout(const IndexLayout &lay, int32_t H_q, bool tables, bool debug);

// Row addressing of a [B][H][n][128] view.
struct KVRows {
    const void *data;
    int64_t sb, sh, sn;   // element strides
    int32_t H;
};

// ---- launchers (return hipSuccess or the launch error) ----
hipError_t launch_wgen(uint64_t seed, int32_t R, int32_t R_pad, float *W, float *Wp, hipStream_t s);
hipError_t launch_mean(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                       int32_t n_mean_blocks, double *mu_part, float *mu, double *mu64,
                       hipStream_t s);
// Encodes keys [256 kb0, n) (whole 256-key blocks; keys >= n are zero rows)
// into planes whose units are nc_cap chunks apart.  With wx non-NULL the
// keys are lifted: projection j gains wx[j] sqrt(r2 - xx_i).
hipError_t launch_encode_keys(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                              int32_t nc_cap, const float *mu, const float *Wp, int32_t K,
                              int32_t L, int32_t R_pad, uint32_t *planes, int32_t kb0,
                              const float *wx, const double *xx, const double *r2, int32_t n_cap,
                              hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, int64_t count, hipStream_t s);
// Codes of keys [n0, n1) of every unit written bit by bit into the planes
// (n1 - n0 <= kAppendMax; K >= 1), with the build's mu and canonical W.
constexpr int kAppendMax = 64;
hipError_t launch_append_codes(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n0,
                               int32_t n1, int32_t nc_cap, const float *mu, const float *W,
                               int32_t K, int32_t L, uint32_t *planes, hipStream_t s);
// The lift: wx from the hyperplane stream; xx, r^2 and r of every unit (mu64
// must hold the fp64 mean).
hipError_t launch_wgen_extra(uint64_t seed, int32_t R, int32_t R_pad, float *wx, hipStream_t s);
hipError_t launch_lift_norms(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                             int32_t n_cap, int32_t nmb, const double *mu64, double *xx,
                             double *xmax, double *r2, float *rnorm, hipStream_t s);

struct DecodeArgs {
    const float *q;          // [BHq][128]
    int32_t B, H_q, H_kv, G, n, n_chunks, K, L, Kr;
    int32_t nc_cap;          // plane chunks per unit (units are this far apart)
    int32_t n_sink, n_local;
    float scale;
    float ucoef[5];          // (L - i + 1) / i for i = 3..7 (0 past L): the binomial tail of log u
    const float *W;          // [R][128]
    const float *mu;         // [B*H_kv][128]
    const float *rnorm;      // [B*H_kv] lift radius r (lifted index) or NULL
    const uint32_t *planes;  // index code planes
    const uint32_t *tab_off; // bucketed tables (table path only)
    const uint32_t *tab_ent;
    uint32_t *bits;          // scratch [BHq][slices][n_pad/16]: 2 bits per key (table path only)
    KVRows k, v;
    int32_t dtype;
    uint16_t *qcodes;        // scratch [BHq][L]
    uint32_t *qq;            // scratch [BHq][L], code | code << 16
    float *qnorm;            // scratch [BHq], |q|
    int32_t app_n0;          // keys [app_n0, n) are appended by this call (app_n0 = n: none)
    uint32_t *app_planes;    // the index's planes, written by that append
    float *part;             // scratch [B*H_kv][n_chunks][G][kD + 2] partial records (a chunk, or a run's chunks of one unit)
    int32_t *unit_cnt;       // scratch [B*H_kv]: records stored per unit, zeroed by the query encode
    int32_t *seg_idx;        // scratch [BHq][n_chunks * kChunk] (debug only)
    int32_t *seg_cnt;        // scratch [BHq][n_chunks] (debug only)
    float *out;              // [BHq][128]
    uint8_t *counts;         // optional [BHq][n] (debug; table path: min(count, 2))
    int32_t *s_idx;          // optional [BHq][n]
    int32_t *s_len;          // optional [BHq]
    bool debug;
    hipEvent_t ev_begin, ev_end;   // optional, recorded around scan_gather
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Records the failure detail for mp_last_error and returns s.
mp_status fail(mp_status s, const char *fmt, ...);
// Validation and launch of every decode entry point (scratch laid out by
// decode_layout(..., tables, debug)).
// n_new >= 0: the call first grows the index from its n to n_new keys (at
// most kAppendMax more, code scan only); the index itself is not changed here.
// check_only: every check, then MP_OK without enqueueing anything (any
// n_new up to the capacity).
mp_status decode_common(const float *q, int32_t H_q, const mp_index *idx, const mp_kv_view *k,
                        const mp_kv_view *v, int32_t n_sink, int32_t n_local, float scale,
                        float *out, void *scratch, size_t scratch_bytes, void *stream, bool debug,
                        uint16_t *qcodes, uint8_t *counts, int32_t *s_idx, int32_t *s_len,
                        void *ev_begin, void *ev_end, bool tables, int32_t n_new = -1,
                        bool check_only = false);
// Scratch bytes of a code-scan decode without the debug lists, or -1 for a
// dead handle or an H_q that does not fit the index.
int64_t decode_scratch_needed(const mp_index *idx, int32_t H_q);
hipError_t launch_encode_query(const DecodeArgs &a, hipStream_t s);
// The LSE merge of the partial records: a unit's records are its runs of cpb
// chunks (cpb = 1: a record per chunk).
hipError_t launch_merge(const DecodeArgs &a, int32_t cpb, hipStream_t s);
hipError_t launch_counts(const DecodeArgs &a, hipStream_t s);
hipError_t launch_seg_compact(const DecodeArgs &a, hipStream_t s);
hipError_t launch_build_tables(const mp_index_impl &idx, hipStream_t s);
hipError_t launch_decode_tables(const DecodeArgs &a, hipStream_t s);

}  // namespace mp
