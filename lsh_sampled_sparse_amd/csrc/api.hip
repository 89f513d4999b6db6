// api.hip -- the C ABI of libmagicpig: argument validation, workspace and
// scratch layouts, and the launch sequence of index build and decode.
// Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <unordered_set>

#include "mp_internal.h"

struct mp_index : mp::mp_index_impl {};

namespace mp {

std::atomic<uint64_t> g_forced_launch_failures{0};

static thread_local char g_err[512] = "";

mp_status fail(mp_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

// The counts that describe the first n keys of an index.
static void set_index_keys(IndexLayout &y, int32_t n)
{
    y.n = n;
    y.n_chunks = ceil_div(n, kChunk);
    y.n_pad = y.n_chunks * kChunk;
    y.n_mean_blocks = ceil_div(n, kMeanRows);
}

IndexLayout index_layout(int32_t B, int32_t H_kv, int32_t n, int32_t K, int32_t L, int32_t n_cap,
                         int32_t flags)
{
    if (n_cap < n) n_cap = n;
    IndexLayout y{};
    y.B = B;
    y.H_kv = H_kv;
    y.n = n_cap;             // regions are sized for n_cap; n is set below
    y.n_chunks = ceil_div(n_cap, kChunk);
    y.n_pad = y.n_chunks * kChunk;
    y.n_mean_blocks = ceil_div(n_cap, kMeanRows);
    y.n_cap = n_cap;
    y.nc_cap = y.n_chunks;
    y.K = K;
    y.L = L;
    y.R = K * L;
    y.R_pad = y.R > 0 ? ceil_div(y.R, 16) * 16 : 16;
    y.Kr = K > 0 ? K : 1;
    const int64_t BH = int64_t(B) * H_kv;
    int64_t off = 0;
    y.off_W = off;       off = align256(off + int64_t(y.R_pad) * kD * 4);
    y.off_Wp = off;      off = align256(off + int64_t(y.R_pad) * kD * 4);
    y.off_mu = off;      off = align256(off + BH * kD * 4);
    y.off_mu_part = off; off = align256(off + BH * y.n_mean_blocks * kD * 8);
    y.off_planes = off;  off = align256(off + BH * y.nc_cap * int64_t(L) * y.Kr * kWords * 4);
    y.flags = flags;
    if (flags & MP_INDEX_MIPS) {
        y.off_wx = off;      off = align256(off + int64_t(y.R_pad) * 4);
        y.off_mu64 = off;    off = align256(off + BH * kD * 8);
        y.off_xx = off;      off = align256(off + BH * int64_t(n_cap) * 8);
        y.off_xmax = off;    off = align256(off + BH * y.n_mean_blocks * 8);
        y.off_r2 = off;      off = align256(off + BH * 8);
        y.off_rn = off;      off = align256(off + BH * 4);
    }
    y.total = off;
    set_index_keys(y, n);
    return y;
}

DecodeLayout decode_layout(const IndexLayout &lay, int32_t H_q, bool tables, bool debug)
{
    DecodeLayout y{};
    y.BHq = lay.B * H_q;
    y.n_chunks = lay.n_chunks;
    const int64_t BHq = y.BHq;
    int64_t off = 0;
    y.off_qcodes = off;  off = align256(off + BHq * lay.L * 2);
    y.off_qq = off;      off = align256(off + BHq * lay.L * 4);
    y.off_qnorm = off;   off = align256(off + BHq * 4);
    y.off_part = off;    off = align256(off + BHq * lay.n_chunks * int64_t(kD + 2) * 4);
    y.off_cnt = off;     off = align256(off + int64_t(lay.B) * lay.H_kv * 4);
    y.off_seg_idx = off;
    if (debug) off = align256(off + BHq * lay.n_chunks * int64_t(kChunk) * 4);
    y.off_seg_cnt = off;
    if (debug) off = align256(off + BHq * lay.n_chunks * 4);
    y.off_bits = off;
    if (tables) off = align256(off + BHq * collide_plan(BHq).slices * (lay.n_pad / 16) * 4);
    y.total = off;
    return y;
}

TablesLayout tables_layout(const IndexLayout &lay)
{
    TablesLayout y{};
    y.nbins = 1 << lay.K;
    const int64_t BH = int64_t(lay.B) * lay.H_kv;
    int64_t off = 0;
    y.off_offsets = off; off = align256(off + BH * lay.L * int64_t(y.nbins + 1) * 4);
    y.off_entries = off; off = align256(off + BH * lay.L * int64_t(lay.n) * 4);
    y.total = off;
    return y;
}

size_t collide_lds_bytes(const IndexLayout &lay)
{
    return size_t(lay.n_pad / 16) * 4 + size_t(2 * lay.L + 1) * 4;
}

// Why the bucketed tables of an index cannot be used, or NULL.
static const char *tables_unsupported(const IndexLayout &lay)
{
    if (lay.K > kMaxTableK) return "tables need K <= 12 (2^K bucket counters in LDS)";
    if (collide_lds_bytes(lay) > kCollideLdsMax)
        return "tables need ceil(n/512)*128 + 4*(2L+1) <= 162,816 (2 bits per key in LDS)";
    return nullptr;
}

static bool sizes_ok(int32_t B, int32_t H, int32_t n, int32_t d, int32_t K, int32_t L)
{
    return B >= 1 && H >= 1 && n >= 1 && n <= MP_MAX_KEYS && d == kD && K >= 0 && K <= 16 &&
           L >= 2 && L <= 255 && int64_t(B) * H <= 65535;
}

static mp_status check_view(const mp_kv_view *v, const char *name)
{
    if (!v) return fail(MP_E_ARG, "%s: view is NULL", name);
    if (!v->data) return fail(MP_E_ARG, "%s: data is NULL", name);
    if (v->dtype != MP_F32 && v->dtype != MP_BF16)
        return fail(MP_E_DTYPE, "%s: dtype %d is not MP_F32 or MP_BF16", name, v->dtype);
    if (v->d != kD) return fail(MP_E_SHAPE, "%s: d = %d, only 128 is supported", name, v->d);
    if (v->B < 1 || v->H < 1 || v->n < 1)
        return fail(MP_E_SHAPE, "%s: B, H, n must be >= 1 (got %d, %d, %d)", name, v->B, v->H, v->n);
    if (v->n > MP_MAX_KEYS)
        return fail(MP_E_SHAPE, "%s: n = %d exceeds MP_MAX_KEYS (%d)", name, v->n, MP_MAX_KEYS);
    if (v->stride_b < 0 || v->stride_h < 0 || v->stride_n < kD)
        return fail(MP_E_SHAPE, "%s: strides must be >= 0 and stride_n >= 128", name);
    const int64_t elt = v->dtype == MP_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(v->data) & 15) || (v->stride_b * elt) % 16 ||
        (v->stride_h * elt) % 16 || (v->stride_n * elt) % 16)
        return fail(MP_E_SHAPE, "%s: data and row strides must be 16-byte aligned", name);
    return MP_OK;
}

// Live index handles.  A handle is looked up here, never dereferenced, before
// it is trusted: a destroyed handle is refused without reading freed memory
// (its address may come back for a later index, which is then the live one).
static std::mutex g_handles_m;
static std::unordered_set<const mp_index *> g_handles;

static void register_handle(const mp_index *idx)
{
    std::lock_guard<std::mutex> g(g_handles_m);
    g_handles.insert(idx);
}

static bool unregister_handle(const mp_index *idx)
{
    std::lock_guard<std::mutex> g(g_handles_m);
    return g_handles.erase(idx) > 0;
}

static const mp_index *live(const mp_index *idx)
{
    if (!idx) return nullptr;
    std::lock_guard<std::mutex> g(g_handles_m);
    return g_handles.count(idx) ? idx : nullptr;
}

mp_status decode_common(const float *q, int32_t H_q, const mp_index *idx, const mp_kv_view *k,
                        const mp_kv_view *v, int32_t n_sink, int32_t n_local, float scale,
                        float *out, void *scratch, size_t scratch_bytes, void *stream, bool debug,
                        uint16_t *qcodes, uint8_t *counts, int32_t *s_idx, int32_t *s_len,
                        void *ev_begin, void *ev_end, bool tables, int32_t n_new,
                        bool check_only)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    // the layout the decode runs on: the index's, or the index grown to n_new
    IndexLayout lay = idx->lay;
    if (n_new >= 0) set_index_keys(lay, n_new);
    if (tables && !idx->tab_off)
        return fail(MP_E_ARG, "the index has no bucketed tables: call mp_build_tables first");
    if (!q || !out) return fail(MP_E_ARG, "q and out must be non-NULL");
    if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(out) & 15))
        return fail(MP_E_ARG, "q and out must be 16-byte aligned");
    if (H_q < 1 || H_q % lay.H_kv)
        return fail(MP_E_SHAPE, "H_q = %d is not a positive multiple of H_kv = %d", H_q, lay.H_kv);
    const int32_t G = H_q / lay.H_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(MP_E_SHAPE, "GQA group size H_q/H_kv = %d; supported: 1, 2, 4, 8", G);
    if (int64_t(lay.B) * H_q > 65535 * 16)
        return fail(MP_E_SHAPE, "B*H_q = %lld is too large", (long long)lay.B * H_q);
    mp_status st = check_view(k, "k");
    if (st != MP_OK) return st;
    st = check_view(v, "v");
    if (st != MP_OK) return st;
    if (k->dtype != v->dtype) return fail(MP_E_DTYPE, "k and v must have the same dtype");
    if (k->dtype != idx->key_dtype)
        return fail(MP_E_DTYPE, "k dtype differs from the keys the index was built from");
    if (k->B != lay.B || k->H != lay.H_kv || k->n != lay.n || v->B != lay.B ||
        v->H != lay.H_kv || v->n != lay.n)
        return fail(MP_E_SHAPE, "k/v shape [%d][%d][%d] / [%d][%d][%d] differs from the index [%d][%d][%d]",
                    k->B, k->H, k->n, v->B, v->H, v->n, lay.B, lay.H_kv, lay.n);
    if (n_sink < 0 || n_local < 0) return fail(MP_E_ARG, "n_sink and n_local must be >= 0");
    if (!isfinite(scale) || scale < 0.0f) return fail(MP_E_ARG, "scale must be finite and >= 0");
    const DecodeLayout dl = decode_layout(lay, H_q, tables, debug);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != idx->device)
        return fail(MP_E_ARG, "current device %d is not the device %d the index lives on", dev,
                    idx->device);
    if (!scratch) return fail(MP_E_WORKSPACE, "scratch is NULL");
    if (reinterpret_cast<uintptr_t>(scratch) & 255)
        return fail(MP_E_WORKSPACE, "scratch must be 256-byte aligned");
    if (scratch_bytes < size_t(dl.total))
        return fail(MP_E_WORKSPACE, "scratch holds %zu bytes, %lld needed", scratch_bytes,
                    (long long)dl.total);
    if (check_only) return MP_OK;

    char *sp = static_cast<char *>(scratch);
    DecodeArgs a{};
    a.q = q;
    a.B = lay.B;
    a.H_q = H_q;
    a.H_kv = lay.H_kv;
    a.G = G;
    a.n = lay.n;
    a.n_chunks = lay.n_chunks;
    a.K = lay.K;
    a.L = lay.L;
    a.n_sink = n_sink;
    a.n_local = n_local;
    a.scale = scale > 0.0f ? scale : 1.0f / sqrtf(float(kD));
    for (int i = 3; i <= 7; ++i)
        a.ucoef[i - 3] = lay.L - i + 1 > 0 ? float(lay.L - i + 1) / float(i) : 0.0f;
    a.W = idx->W;
    a.mu = idx->mu;
    a.rnorm = idx->rnorm;
    a.planes = idx->planes;
    a.Kr = lay.Kr;
    a.nc_cap = lay.nc_cap;
    a.k = KVRows{k->data, k->stride_b, k->stride_h, k->stride_n, k->H};
    a.v = KVRows{v->data, v->stride_b, v->stride_h, v->stride_n, v->H};
    a.dtype = k->dtype;
    a.qcodes = reinterpret_cast<uint16_t *>(sp + dl.off_qcodes);
    a.qq = reinterpret_cast<uint32_t *>(sp + dl.off_qq);
    a.qnorm = reinterpret_cast<float *>(sp + dl.off_qnorm);
    a.app_n0 = n_new >= 0 ? idx->lay.n : lay.n;
    a.app_planes = idx->planes;
    a.part = reinterpret_cast<float *>(sp + dl.off_part);
    a.unit_cnt = reinterpret_cast<int32_t *>(sp + dl.off_cnt);
    a.seg_idx = reinterpret_cast<int32_t *>(sp + dl.off_seg_idx);
    a.seg_cnt = reinterpret_cast<int32_t *>(sp + dl.off_seg_cnt);
    a.tab_off = idx->tab_off;
    a.tab_ent = idx->tab_ent;
    a.bits = tables ? reinterpret_cast<uint32_t *>(sp + dl.off_bits) : nullptr;
    a.out = out;
    a.counts = counts;
    a.s_idx = s_idx;
    a.s_len = s_len;
    a.debug = debug;
    a.ev_begin = static_cast<hipEvent_t>(ev_begin);
    a.ev_end = static_cast<hipEvent_t>(ev_end);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = tables ? launch_decode_tables(a, s) : launch_decode(a, s);
    if (e != hipSuccess) return fail(MP_E_HIP, "decode launch failed: %s", hipGetErrorString(e));
    if (debug && qcodes) {
        e = hipMemcpyAsync(qcodes, a.qcodes, size_t(dl.BHq) * lay.L * 2, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return fail(MP_E_HIP, "qcodes copy failed: %s", hipGetErrorString(e));
    }
    return MP_OK;
}

int64_t decode_scratch_needed(const mp_index *idx, int32_t H_q)
{
    if (!live(idx) || H_q < 1 || H_q % idx->lay.H_kv) return -1;
    return decode_layout(idx->lay, H_q, false, false).total;
}

}  // namespace mp

using namespace mp;

extern "C" {

size_t mp_index_workspace_bytes_ex(int32_t B, int32_t H_kv, int32_t n, int32_t d, int32_t K,
                                   int32_t L, int32_t flags)
{
    if (!sizes_ok(B, H_kv, n, d, K, L) || (flags & ~MP_INDEX_MIPS)) return 0;
    return size_t(index_layout(B, H_kv, n, K, L, n, flags).total);
}

size_t mp_index_workspace_bytes(int32_t B, int32_t H_kv, int32_t n, int32_t d, int32_t K, int32_t L)
{
    return mp_index_workspace_bytes_ex(B, H_kv, n, d, K, L, 0);
}

static mp_status build_index_impl(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                                  int32_t n_cap, int32_t flags, void *workspace,
                                  size_t workspace_bytes, void *stream, mp_index **out)
{
    g_err[0] = 0;
    if (!out) return fail(MP_E_ARG, "out is NULL");
    *out = nullptr;
    mp_status st = check_view(keys, "keys");
    if (st != MP_OK) return st;
    if (K < 0 || K > 16) return fail(MP_E_ARG, "K = %d outside [0, 16]", K);
    if (L < 2 || L > 255) return fail(MP_E_ARG, "L = %d outside [2, 255]", L);
    if (int64_t(keys->B) * keys->H > 65535)
        return fail(MP_E_SHAPE, "B*H_kv = %lld is too large", (long long)keys->B * keys->H);
    if (flags & ~MP_INDEX_MIPS) return fail(MP_E_ARG, "unknown build flags 0x%x", flags);
    if (n_cap < keys->n) return fail(MP_E_ARG, "capacity %d is below the %d keys", n_cap, keys->n);
    if (mp_index_workspace_bytes(keys->B, keys->H, n_cap, keys->d, K, L) == 0)
        return fail(MP_E_ARG, "capacity %d is not a valid key count", n_cap);
    const IndexLayout lay = index_layout(keys->B, keys->H, keys->n, K, L, n_cap, flags);
    if (!workspace) return fail(MP_E_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255)
        return fail(MP_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < size_t(lay.total))
        return fail(MP_E_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                    (long long)lay.total);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MP_E_HIP, "no current HIP device");

    mp_index *idx = new (std::nothrow) mp_index();
    if (!idx) return fail(MP_E_ARG, "host allocation of the handle failed");
    char *wp = static_cast<char *>(workspace);
    idx->lay = lay;
    idx->seed = seed;
    idx->key_dtype = keys->dtype;
    idx->device = dev;
    idx->W = reinterpret_cast<float *>(wp + lay.off_W);
    idx->Wp = reinterpret_cast<float *>(wp + lay.off_Wp);
    idx->mu = reinterpret_cast<float *>(wp + lay.off_mu);
    idx->mu_part = reinterpret_cast<double *>(wp + lay.off_mu_part);
    idx->planes = reinterpret_cast<uint32_t *>(wp + lay.off_planes);
    const bool lift = flags & MP_INDEX_MIPS;
    if (lift) {
        idx->wx = reinterpret_cast<float *>(wp + lay.off_wx);
        idx->mu64 = reinterpret_cast<double *>(wp + lay.off_mu64);
        idx->xx = reinterpret_cast<double *>(wp + lay.off_xx);
        idx->xmax = reinterpret_cast<double *>(wp + lay.off_xmax);
        idx->r2 = reinterpret_cast<double *>(wp + lay.off_r2);
        idx->rnorm = reinterpret_cast<float *>(wp + lay.off_rn);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    const KVRows rows{keys->data, keys->stride_b, keys->stride_h, keys->stride_n, keys->H};
    hipError_t e = launch_wgen(seed, lay.R, lay.R_pad, idx->W, idx->Wp, s);
    if (e == hipSuccess && lift) e = launch_wgen_extra(seed, lay.R, lay.R_pad, idx->wx, s);
    if (e == hipSuccess)
        e = launch_mean(rows, keys->dtype, lay.B, lay.H_kv, lay.n, lay.n_mean_blocks, idx->mu_part,
                        idx->mu, idx->mu64, s);
    if (e == hipSuccess && lift)
        e = launch_lift_norms(rows, keys->dtype, lay.B, lay.H_kv, lay.n, lay.n_cap,
                              lay.n_mean_blocks, idx->mu64, idx->xx, idx->xmax, idx->r2,
                              idx->rnorm, s);
    if (e == hipSuccess) {
        const int64_t nwords = int64_t(lay.B) * lay.H_kv * lay.nc_cap * int64_t(L) * lay.Kr * kWords;
        if (K == 0)
            e = launch_fill_u32(idx->planes, nwords, s);   // every code is 0: one zero row per table
        else
            e = launch_encode_keys(rows, keys->dtype, lay.B, lay.H_kv, lay.n, lay.nc_cap, idx->mu,
                                   idx->Wp, K, L, lay.R_pad, idx->planes, 0, idx->wx, idx->xx,
                                   idx->r2, lay.n_cap, s);
    }
    if (e != hipSuccess) {
        delete idx;
        return fail(MP_E_HIP, "index build launch failed: %s", hipGetErrorString(e));
    }
    register_handle(idx);
    *out = idx;
    return MP_OK;
}

mp_status mp_build_index(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                         void *workspace, size_t workspace_bytes, void *stream, mp_index **out)
{
    return build_index_impl(keys, K, L, seed, keys ? keys->n : 0, 0, workspace, workspace_bytes,
                            stream, out);
}

mp_status mp_build_index_cap(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                             int32_t n_cap, void *workspace, size_t workspace_bytes, void *stream,
                             mp_index **out)
{
    return build_index_impl(keys, K, L, seed, n_cap, 0, workspace, workspace_bytes, stream, out);
}

mp_status mp_build_index_ex(const mp_kv_view *keys, int32_t K, int32_t L, uint64_t seed,
                            int32_t n_cap, int32_t flags, void *workspace, size_t workspace_bytes,
                            void *stream, mp_index **out)
{
    return build_index_impl(keys, K, L, seed, n_cap, flags, workspace, workspace_bytes, stream,
                            out);
}

mp_status mp_index_lift_views(const mp_index *idx, const float **w_extra, const float **r)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    if (!(idx->lay.flags & MP_INDEX_MIPS)) return fail(MP_E_ARG, "the index has no lift");
    if (w_extra) *w_extra = idx->wx;
    if (r) *r = idx->rnorm;
    return MP_OK;
}

mp_status mp_index_append(mp_index *idx, const mp_kv_view *keys, void *stream)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    IndexLayout &lay = idx->lay;
    if (lay.flags & MP_INDEX_MIPS)
        return fail(MP_E_ARG, "a lifted index cannot grow: its radius covers the built keys");
    mp_status st = check_view(keys, "keys");
    if (st != MP_OK) return st;
    if (keys->dtype != idx->key_dtype) return fail(MP_E_DTYPE, "keys dtype differs from the index's");
    if (keys->B != lay.B || keys->H != lay.H_kv)
        return fail(MP_E_SHAPE, "keys are [%d][%d][...], the index covers [%d][%d]", keys->B,
                    keys->H, lay.B, lay.H_kv);
    if (keys->n < lay.n)
        return fail(MP_E_SHAPE, "keys hold %d keys, fewer than the index's %d", keys->n, lay.n);
    if (keys->n > lay.n_cap)
        return fail(MP_E_SHAPE, "%d keys exceed the index capacity %d", keys->n, lay.n_cap);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != idx->device)
        return fail(MP_E_ARG, "the current device is not the index's device");
    if (keys->n == lay.n) return MP_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (lay.K > 0) {
        const KVRows rows{keys->data, keys->stride_b, keys->stride_h, keys->stride_n, keys->H};
        hipError_t e;
        if (keys->n - lay.n <= kAppendMax) {
            // a few keys: their bits alone, written into the plane words
            e = launch_append_codes(rows, keys->dtype, lay.B, lay.H_kv, lay.n, keys->n, lay.nc_cap,
                                    idx->mu, idx->W, lay.K, lay.L, idx->planes, s);
        } else {
            // from the 256-key block holding the first new key: its old keys
            // are encoded again to the same bits, so every plane word is
            // written whole
            e = launch_encode_keys(rows, keys->dtype, lay.B, lay.H_kv, keys->n, lay.nc_cap,
                                   idx->mu, idx->Wp, lay.K, lay.L, lay.R_pad, idx->planes,
                                   lay.n / 256, nullptr, nullptr, nullptr, lay.n_cap, s);
        }
        if (e != hipSuccess)
            return fail(MP_E_HIP, "append launch failed: %s", hipGetErrorString(e));
    }
    set_index_keys(lay, keys->n);
    idx->tab_off = nullptr;    // tables of the old keys no longer describe the index
    idx->tab_ent = nullptr;
    return MP_OK;
}

size_t mp_decode_scratch_bytes(const mp_index *idx, int32_t H_q)
{
    if (!live(idx) || H_q < 1 || H_q % idx->lay.H_kv) return 0;
    IndexLayout cap = idx->lay;   // grown to its capacity: one scratch serves every size
    set_index_keys(cap, cap.n_cap);
    return size_t(decode_layout(cap, H_q, false, true).total);
}

mp_status mp_decode_attn(const float *q, int32_t H_q, const mp_index *idx, const mp_kv_view *k,
                         const mp_kv_view *v, int32_t n_sink, int32_t n_local, float scale,
                         float *out, void *scratch, size_t scratch_bytes, void *stream)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false);
}

mp_status mp_decode_attn_append(const float *q, int32_t H_q, mp_index *idx, const mp_kv_view *k,
                                const mp_kv_view *v, int32_t n_sink, int32_t n_local, float scale,
                                float *out, void *scratch, size_t scratch_bytes, void *stream)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    const IndexLayout &lay = idx->lay;
    mp_status st = check_view(k, "k");
    if (st != MP_OK) return st;
    if (k->n == lay.n)   // nothing to add
        return mp_decode_attn(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch,
                              scratch_bytes, stream);
    if (lay.flags & MP_INDEX_MIPS)
        return fail(MP_E_ARG, "an index built with MP_INDEX_MIPS does not grow");
    if (k->n < lay.n)
        return fail(MP_E_SHAPE, "k holds %d keys, fewer than the %d indexed", k->n, lay.n);
    if (k->n > lay.n_cap)
        return fail(MP_E_SHAPE, "%d keys exceed the index capacity %d", k->n, lay.n_cap);
    // every argument of the decode over the grown index, before anything changes
    st = decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                       stream, false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false,
                       k->n, true);
    if (st != MP_OK) return st;
    if (k->n - lay.n > kAppendMax || lay.K == 0) {
        // many keys, or no bits to write: the two calls
        st = mp_index_append(idx, k, stream);
        if (st != MP_OK) return st;
        return mp_decode_attn(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch,
                              scratch_bytes, stream);
    }
    // 1 to kAppendMax new keys: their codes ride on the decode's query encode
    st = decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                       stream, false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false,
                       k->n);
    if (st != MP_OK) return st;
    set_index_keys(idx->lay, k->n);
    idx->tab_off = nullptr;    // tables of the old keys no longer describe the index
    idx->tab_ent = nullptr;
    return MP_OK;
}

mp_status mp_decode_attn_timed(const float *q, int32_t H_q, const mp_index *idx,
                               const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                               int32_t n_local, float scale, float *out, void *scratch,
                               size_t scratch_bytes, void *stream, void *ev_scan_begin,
                               void *ev_scan_end)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, false, nullptr, nullptr, nullptr, nullptr, ev_scan_begin,
                         ev_scan_end, false);
}

mp_status mp_decode_debug(const float *q, int32_t H_q, const mp_index *idx, const mp_kv_view *k,
                          const mp_kv_view *v, int32_t n_sink, int32_t n_local, float scale,
                          float *out, void *scratch, size_t scratch_bytes, void *stream,
                          uint16_t *qcodes, uint8_t *counts, int32_t *s_idx, int32_t *s_len)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, true, qcodes, counts, s_idx, s_len, nullptr, nullptr, false);
}

size_t mp_tables_workspace_bytes(const mp_index *idx)
{
    if (!live(idx) || tables_unsupported(idx->lay)) return 0;
    return size_t(tables_layout(idx->lay).total);
}

mp_status mp_build_tables(mp_index *idx, void *workspace, size_t workspace_bytes, void *stream)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    if (const char *why = tables_unsupported(idx->lay)) return fail(MP_E_SHAPE, "%s", why);
    const TablesLayout tl = tables_layout(idx->lay);
    if (!workspace) return fail(MP_E_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) & 255)
        return fail(MP_E_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < size_t(tl.total))
        return fail(MP_E_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                    (long long)tl.total);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != idx->device)
        return fail(MP_E_ARG, "current device %d is not the device %d the index lives on", dev,
                    idx->device);
    char *wp = static_cast<char *>(workspace);
    idx->tab_off = reinterpret_cast<uint32_t *>(wp + tl.off_offsets);
    idx->tab_ent = reinterpret_cast<uint32_t *>(wp + tl.off_entries);
    const hipError_t e = launch_build_tables(*idx, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        idx->tab_off = idx->tab_ent = nullptr;
        return fail(MP_E_HIP, "table build launch failed: %s", hipGetErrorString(e));
    }
    return MP_OK;
}

size_t mp_decode_tables_scratch_bytes(const mp_index *idx, int32_t H_q)
{
    if (!live(idx) || H_q < 1 || H_q % idx->lay.H_kv || tables_unsupported(idx->lay)) return 0;
    return size_t(decode_layout(idx->lay, H_q, true, true).total);
}

mp_status mp_decode_attn_tables(const float *q, int32_t H_q, const mp_index *idx,
                                const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                int32_t n_local, float scale, float *out, void *scratch,
                                size_t scratch_bytes, void *stream)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true);
}

mp_status mp_decode_attn_tables_timed(const float *q, int32_t H_q, const mp_index *idx,
                                      const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                      int32_t n_local, float scale, float *out, void *scratch,
                                      size_t scratch_bytes, void *stream, void *ev_gather_begin,
                                      void *ev_gather_end)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, false, nullptr, nullptr, nullptr, nullptr, ev_gather_begin,
                         ev_gather_end, true);
}

mp_status mp_decode_tables_debug(const float *q, int32_t H_q, const mp_index *idx,
                                 const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                 int32_t n_local, float scale, float *out, void *scratch,
                                 size_t scratch_bytes, void *stream, uint16_t *qcodes,
                                 uint8_t *counts2, int32_t *s_idx, int32_t *s_len)
{
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, scratch, scratch_bytes,
                         stream, true, qcodes, counts2, s_idx, s_len, nullptr, nullptr, true);
}

mp_status mp_tables_views(const mp_index *idx, const uint32_t **offsets, const uint32_t **entries)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    if (!idx->tab_off) return fail(MP_E_ARG, "the index has no bucketed tables");
    if (offsets) *offsets = idx->tab_off;
    if (entries) *entries = idx->tab_ent;
    return MP_OK;
}

mp_status mp_index_views(const mp_index *idx, const float **W, const float **mu,
                         const uint32_t **planes, int32_t *n_pad)
{
    g_err[0] = 0;
    if (!live(idx)) return fail(MP_E_HANDLE, "index handle is NULL or not a live index");
    if (W) *W = idx->W;
    if (mu) *mu = idx->mu;
    if (planes) *planes = idx->planes;
    if (n_pad) *n_pad = idx->lay.n_pad;
    return MP_OK;
}

void mp_index_destroy(mp_index *idx)
{
    if (idx && unregister_handle(idx)) delete idx;
}

void mp_debug_fail_launches(int32_t skip, int32_t count)
{
    const uint64_t c = count > 0 ? uint64_t(count) : 0, k = skip > 0 && c ? uint64_t(skip) : 0;
    g_forced_launch_failures.store(k << 32 | c, std::memory_order_relaxed);
}

const char *mp_status_str(mp_status s)
{
    switch (s) {
    case MP_OK: return "MP_OK";
    case MP_E_ARG: return "MP_E_ARG: invalid argument";
    case MP_E_SHAPE: return "MP_E_SHAPE: unsupported or mismatched shape";
    case MP_E_DTYPE: return "MP_E_DTYPE: unsupported dtype";
    case MP_E_WORKSPACE: return "MP_E_WORKSPACE: workspace or scratch too small or misaligned";
    case MP_E_HIP: return "MP_E_HIP: HIP call or kernel launch failed";
    case MP_E_HANDLE: return "MP_E_HANDLE: not a live index";
    }
    return "unknown mp_status";
}

const char *mp_last_error(void) { return g_err; }

}  // extern "C"
