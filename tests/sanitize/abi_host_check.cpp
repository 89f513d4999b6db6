// abi_host_check.cpp -- the host half of libmagicpig under AddressSanitizer +
// UndefinedBehaviorSanitizer, or ThreadSanitizer (g++ on the CPU, no GPU).
//
// TEST INFRASTRUCTURE: built and run by tests/test_sanitize_cpu.py.
//
// The library's C-ABI source (argument validation, the handle registry, the
// workspace and scratch layouts, the launch sequences) is compiled here with
// the host compiler.  Every kernel launcher it calls, and the three HIP runtime
// calls it makes, are replaced by stand-ins that check the launch arguments
// against the shapes and then touch every byte of every region the kernels
// would read or write, sized from the shapes alone (not from the layouts).
// Buffers are allocated with exactly the sizes the library's *_bytes queries
// return, so a region laid out past the end of its buffer, or a size query
// that comes up short, is a heap-buffer-overflow report; a handle used after
// mp_index_destroy is a use-after-free report; an index the library forgets to
// free is a leak report.
//
// Usage: abi_host_check [all|threads]   (exit status 0 when every check holds)

// hip_ext.h's launch templates need the HIP compiler; the C-ABI source
// launches nothing itself (the launchers below stand in for the kernels).
#define HIP_INCLUDE_HIP_HIP_EXT_H
#include "../../lsh_sampled_sparse_amd/csrc/api.hip"

#include <stdlib.h>

#include <thread>
#include <vector>

// ---------------------------------------------------------------- checks ----

static int g_failed = 0;

#define EXPECT(c)                                                                        \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);               \
            ++g_failed;                                                                  \
        }                                                                                \
    } while (0)

#define EXPECT_ST(call, want)                                                            \
    do {                                                                                 \
        const mp_status got_ = (call);                                                   \
        if (got_ != (want)) {                                                            \
            fprintf(stderr, "FAILED %s:%d: %s returned %s (%s), expected %s\n", __FILE__, \
                    __LINE__, #call, mp_status_str(got_), mp_last_error(), #want);       \
            ++g_failed;                                                                  \
        } else if (got_ != MP_OK && mp_last_error()[0] == 0) {                           \
            fprintf(stderr, "FAILED %s:%d: %s gave no error text\n", __FILE__, __LINE__,  \
                    #call);                                                              \
            ++g_failed;                                                                  \
        }                                                                                \
    } while (0)

// ------------------------------------------------ touching device regions ----

static void rd(const void *p, int64_t bytes)
{
    if (bytes <= 0) return;
    if (!p) {
        fprintf(stderr, "FAILED: a launch reads %lld bytes through a NULL pointer\n",
                (long long)bytes);
        ++g_failed;
        return;
    }
    static thread_local char sink[1 << 16];
    const char *c = static_cast<const char *>(p);
    for (int64_t o = 0; o < bytes; o += sizeof sink) {
        const int64_t m = bytes - o < int64_t(sizeof sink) ? bytes - o : int64_t(sizeof sink);
        memcpy(sink, c + o, size_t(m));   // the interceptor checks the whole range
    }
}

static void wr(void *p, int64_t bytes)
{
    if (bytes <= 0) return;
    if (!p) {
        fprintf(stderr, "FAILED: a launch writes %lld bytes through a NULL pointer\n",
                (long long)bytes);
        ++g_failed;
        return;
    }
    memset(p, 0xA5, size_t(bytes));
}

// Rows [i0, i1) of every (sequence, head) of a [B][H][n][128] view.
static void rd_rows(const mp::KVRows &r, int32_t dtype, int32_t B, int32_t H, int32_t i0,
                    int32_t i1)
{
    const int64_t elt = dtype == MP_F32 ? 4 : 2;
    EXPECT(r.H == H);
    for (int32_t b = 0; b < B; ++b)
        for (int32_t h = 0; h < H; ++h)
            for (int32_t i = i0; i < i1; ++i)
                rd(static_cast<const char *>(r.data) + (b * r.sb + h * r.sh + i * r.sn) * elt,
                   128 * elt);
}

// ------------------------------------- stand-ins for the HIP runtime calls ----

static int g_device = 0;

hipError_t hipGetDevice(int *dev)
{
    *dev = g_device;
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t)
{
    memcpy(dst, src, bytes);
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t e)
{
    return e == hipSuccess ? "no error" : "launch failure (stand-in)";
}

// ------------------------------------------ stand-ins for the launchers ----

namespace mp {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_wgen(uint64_t, int32_t R, int32_t R_pad, float *W, float *Wp, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(R >= 0 && R <= R_pad && R_pad % 16 == 0 && R_pad >= 16);
    wr(W, int64_t(R_pad) * 128 * 4);
    wr(Wp, int64_t(R_pad) * 128 * 4);
    return hipSuccess;
}

hipError_t launch_wgen_extra(uint64_t, int32_t R, int32_t R_pad, float *wx, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(R <= R_pad);
    wr(wx, int64_t(R_pad) * 4);
    return hipSuccess;
}

hipError_t launch_mean(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                       int32_t nmb, double *mu_part, float *mu, double *mu64, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(nmb == cdiv(n, 1024));
    const int64_t BH = int64_t(B) * H;
    rd_rows(keys, dtype, B, H, 0, n);
    wr(mu_part, BH * nmb * 128 * 8);
    wr(mu, BH * 128 * 4);
    if (mu64) wr(mu64, BH * 128 * 8);
    return hipSuccess;
}

hipError_t launch_lift_norms(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                             int32_t n_cap, int32_t nmb, const double *mu64, double *xx,
                             double *xmax, double *r2, float *rnorm, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(n <= n_cap && nmb == cdiv(n, 1024));
    const int64_t BH = int64_t(B) * H;
    rd_rows(keys, dtype, B, H, 0, n);
    rd(mu64, BH * 128 * 8);
    wr(xx, BH * n_cap * 8);
    wr(xmax, BH * nmb * 8);
    wr(r2, BH * 8);
    wr(rnorm, BH * 4);
    return hipSuccess;
}

// Planes of a unit: nc_cap chunks x L*K rows x 16 words.
hipError_t launch_encode_keys(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                              int32_t nc_cap, const float *mu, const float *Wp, int32_t K,
                              int32_t L, int32_t R_pad, uint32_t *planes, int32_t kb0,
                              const float *wx, const double *xx, const double *r2, int32_t n_cap,
                              hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(K >= 1 && K * L <= R_pad && n <= n_cap && nc_cap == cdiv(n_cap, 512));
    EXPECT(kb0 >= 0 && int64_t(kb0) * 256 < n);
    const int64_t BH = int64_t(B) * H;
    rd_rows(keys, dtype, B, H, kb0 * 256, n);
    rd(mu, BH * 128 * 4);
    rd(Wp, int64_t(R_pad) * 128 * 4);
    if (wx) {
        rd(wx, int64_t(R_pad) * 4);
        rd(xx, BH * n_cap * 8);
        rd(r2, BH * 8);
    }
    // whole 256-key blocks from kb0 on; a chunk's row words cover 512 keys
    const int64_t c0 = int64_t(kb0) * 256 / 512, c1 = cdiv(cdiv(n, 256) * 256, 512);
    EXPECT(c1 <= nc_cap);
    const int64_t chunk_words = int64_t(L) * K * 16;
    for (int64_t u = 0; u < BH; ++u)
        wr(planes + (u * nc_cap + c0) * chunk_words, (c1 - c0) * chunk_words * 4);
    return hipSuccess;
}

hipError_t launch_append_codes(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n0,
                               int32_t n1, int32_t nc_cap, const float *mu, const float *W,
                               int32_t K, int32_t L, uint32_t *planes, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    EXPECT(K >= 1 && n0 < n1 && n1 - n0 <= kAppendMax && n1 <= int64_t(nc_cap) * 512);
    const int64_t BH = int64_t(B) * H;
    rd_rows(keys, dtype, B, H, n0, n1);
    rd(mu, BH * 128 * 4);
    rd(W, int64_t(K) * L * 128 * 4);
    // each row's words holding the new keys, in every unit
    const int64_t chunk_words = int64_t(L) * K * 16;
    for (int64_t u = 0; u < BH; ++u)
        for (int64_t i = n0; i < n1; ++i)
            for (int64_t r = 0; r < int64_t(K) * L; ++r)
                wr(planes + (u * nc_cap + i / 512) * chunk_words + r * 16 + (i % 512) / 32, 4);
    return hipSuccess;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t count, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    wr(p, count * 4);
    return hipSuccess;
}

static void check_decode_args(const DecodeArgs &a, bool tables)
{
    const int64_t BH = int64_t(a.B) * a.H_kv, BHq = int64_t(a.B) * a.H_q;
    const int64_t n_pad = int64_t(a.n_chunks) * 512;
    EXPECT(a.G * a.H_kv == a.H_q && a.n_chunks == cdiv(a.n, 512) && a.n_chunks <= a.nc_cap);
    EXPECT(a.scale > 0.0f && a.Kr == (a.K > 0 ? a.K : 1));
    for (int i = 3; i <= 7; ++i)
        EXPECT(a.ucoef[i - 3] == (a.L - i + 1 > 0 ? float(a.L - i + 1) / float(i) : 0.0f));
    // inputs
    rd(a.q, BHq * 128 * 4);
    rd(a.W, int64_t(a.K) * a.L * 128 * 4);
    rd(a.mu, BH * 128 * 4);
    if (a.rnorm) rd(a.rnorm, BH * 4);
    rd_rows(a.k, a.dtype, a.B, a.H_kv, 0, a.n);
    rd_rows(a.v, a.dtype, a.B, a.H_kv, 0, a.n);
    if (tables) {
        rd(a.tab_off, BH * a.L * ((int64_t(1) << a.K) + 1) * 4);
        rd(a.tab_ent, BH * a.L * int64_t(a.n) * 4);
        wr(a.bits, BHq * collide_plan(BHq).slices * (n_pad / 16) * 4);
    } else {
        rd(a.planes, BH * a.nc_cap * a.L * a.Kr * 16 * 4);
        EXPECT(a.bits == nullptr);
    }
    // keys [app_n0, n) appended by the call: their words of the index's planes
    EXPECT(a.app_n0 <= a.n && a.n - a.app_n0 <= kAppendMax);
    if (a.app_n0 < a.n) {
        EXPECT(!tables && a.K > 0 && a.app_n0 >= 0 && a.app_planes == a.planes);
        wr(a.app_planes, BH * a.nc_cap * a.L * a.K * 16 * 4);
    }
    // scratch and outputs
    wr(a.qcodes, BHq * a.L * 2);
    wr(a.qq, BHq * a.L * 4);
    wr(a.qnorm, BHq * 4);
    wr(a.part, BH * a.n_chunks * a.G * (128 + 2) * 4);
    wr(a.unit_cnt, BH * 4);
    if (a.debug) {
        wr(a.seg_idx, BHq * n_pad * 4);
        wr(a.seg_cnt, BHq * a.n_chunks * 4);
    }
    if (a.counts) wr(a.counts, BHq * a.n);
    if (a.s_idx) wr(a.s_idx, BHq * a.n * 4);
    if (a.s_len) wr(a.s_len, BHq * 4);
    wr(a.out, BHq * 128 * 4);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    check_decode_args(a, false);
    return hipSuccess;
}

hipError_t launch_decode_tables(const DecodeArgs &a, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    check_decode_args(a, true);
    return hipSuccess;
}

hipError_t launch_build_tables(const mp_index_impl &idx, hipStream_t)
{
    if (take_forced_failure()) return hipErrorLaunchFailure;
    const IndexLayout &y = idx.lay;
    const int64_t BH = int64_t(y.B) * y.H_kv;
    EXPECT(y.K <= kMaxTableK);
    rd(idx.planes, BH * y.nc_cap * y.L * y.Kr * 16 * 4);
    wr(idx.tab_off, BH * y.L * ((int64_t(1) << y.K) + 1) * 4);
    wr(idx.tab_ent, BH * y.L * int64_t(y.n) * 4);
    return hipSuccess;
}

}  // namespace mp

// -------------------------------------------------------------- buffers ----

// A host buffer of exactly `bytes` bytes, 256-byte aligned (the sanitizer
// tracks the requested size, so one byte past the end is reported).
struct Buf {
    void *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n(bytes)
    {
        if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) p = nullptr;
        if (p) memset(p, 0, bytes);
    }
    ~Buf() { free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
    template <typename T> T *as() const { return static_cast<T *>(p); }
};

// A [B][H][n][128] tensor with row pitch `pitch` elements (>= 128).
struct KV {
    Buf buf;
    mp_kv_view view;
    KV(int32_t dtype, int32_t B, int32_t H, int32_t n, int64_t pitch = 128)
        : buf(size_t(B) * H * n * pitch * (dtype == MP_F32 ? 4 : 2))
    {
        view.data = buf.p;
        view.dtype = dtype;
        view.B = B;
        view.H = H;
        view.n = n;
        view.d = 128;
        view.stride_n = pitch;
        view.stride_h = int64_t(n) * pitch;
        view.stride_b = int64_t(H) * n * pitch;
    }
    // the first m keys of each (sequence, head)
    mp_kv_view prefix(int32_t m) const
    {
        mp_kv_view v = view;
        v.n = m;
        return v;
    }
};

// --------------------------------------------------------- success paths ----

struct Case {
    const char *name;
    int32_t dtype, B, H_kv, n, K, L, G, n_cap, flags, grow_to;
    int64_t pitch;
};

static void run_case(const Case &c)
{
    printf("case %s\n", c.name);
    fflush(stdout);
    const int32_t n_all = c.grow_to > c.n ? c.grow_to : c.n;
    const int32_t n_cap = c.n_cap > 0 ? c.n_cap : c.n;
    KV keys(c.dtype, c.B, c.H_kv, n_all, c.pitch), vals(c.dtype, c.B, c.H_kv, n_all, c.pitch);
    mp_kv_view kv = keys.prefix(c.n), vv = vals.prefix(c.n);

    const size_t ws = mp_index_workspace_bytes_ex(c.B, c.H_kv, n_cap, 128, c.K, c.L, c.flags);
    EXPECT(ws > 0);
    Buf w(ws);
    mp_index *idx = nullptr;
    EXPECT_ST(mp_build_index_ex(&kv, c.K, c.L, 7, n_cap, c.flags, w.p, ws - 1, nullptr, &idx),
              MP_E_WORKSPACE);
    EXPECT(idx == nullptr);
    EXPECT_ST(mp_build_index_ex(&kv, c.K, c.L, 7, n_cap, c.flags, w.p, ws, nullptr, &idx), MP_OK);
    if (!idx) return;
    if (c.flags == 0 && n_cap == c.n)
        EXPECT(mp_index_workspace_bytes(c.B, c.H_kv, c.n, 128, c.K, c.L) == ws);

    const int32_t H_q = c.G * c.H_kv;
    const int64_t BHq = int64_t(c.B) * H_q;
    Buf q(size_t(BHq) * 128 * 4), out(size_t(BHq) * 128 * 4), s_len(size_t(BHq) * 4);
    Buf qcodes(size_t(BHq) * c.L * 2);

    auto decode_all = [&](int32_t n) {
        Buf counts(size_t(BHq) * n), s_idx(size_t(BHq) * n * 4);
        // production decode: exactly the bytes it needs
        const int64_t need = mp::decode_scratch_needed(idx, H_q);
        EXPECT(need > 0);
        {
            Buf sc{size_t(need)};
            EXPECT_ST(mp_decode_attn(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                     out.as<float>(), sc.p, sc.n - 1, nullptr),
                      MP_E_WORKSPACE);
            EXPECT_ST(mp_decode_attn(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                     out.as<float>(), sc.p, sc.n, nullptr),
                      MP_OK);
            int ev0 = 0, ev1 = 0;   // opaque to the host code: passed through to the launch
            EXPECT_ST(mp_decode_attn_timed(q.as<float>(), H_q, idx, &kv, &vv, 0, 0, 0.5f,
                                           out.as<float>(), sc.p, sc.n, nullptr, &ev0, &ev1),
                      MP_OK);
        }
        // debug decode: mp_decode_scratch_bytes covers it
        const size_t dbytes = mp_decode_scratch_bytes(idx, H_q);
        EXPECT(dbytes >= size_t(need));
        {
            Buf sc(dbytes);
            EXPECT_ST(mp_decode_debug(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                      out.as<float>(), sc.p, sc.n, nullptr, qcodes.as<uint16_t>(),
                                      counts.as<uint8_t>(), s_idx.as<int32_t>(),
                                      s_len.as<int32_t>()),
                      MP_OK);
            EXPECT_ST(mp_decode_debug(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                      out.as<float>(), sc.p, sc.n, nullptr, nullptr, nullptr,
                                      nullptr, nullptr),
                      MP_OK);
        }
        // bucketed tables, where the index allows them
        const size_t tw = mp_tables_workspace_bytes(idx);
        if (tw == 0) {
            EXPECT_ST(mp_build_tables(idx, w.p, 1 << 20, nullptr), MP_E_SHAPE);
            return;
        }
        Buf t(tw);
        EXPECT_ST(mp_decode_attn_tables(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                        out.as<float>(), t.p, t.n, nullptr),
                  MP_E_ARG);   // no tables yet
        EXPECT_ST(mp_build_tables(idx, t.p, tw - 1, nullptr), MP_E_WORKSPACE);
        EXPECT_ST(mp_build_tables(idx, t.p, tw, nullptr), MP_OK);
        const uint32_t *offs = nullptr, *ents = nullptr;
        EXPECT_ST(mp_tables_views(idx, &offs, &ents), MP_OK);
        EXPECT(offs == t.p);
        const size_t tsb = mp_decode_tables_scratch_bytes(idx, H_q);
        EXPECT(tsb > 0);
        Buf sc(tsb);
        EXPECT_ST(mp_decode_attn_tables(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                        out.as<float>(), sc.p, sc.n, nullptr),
                  MP_OK);
        int ev0 = 0, ev1 = 0;
        EXPECT_ST(mp_decode_attn_tables_timed(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                              out.as<float>(), sc.p, sc.n, nullptr, &ev0, &ev1),
                  MP_OK);
        Buf counts2(size_t(BHq) * n);
        EXPECT_ST(mp_decode_tables_debug(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                         out.as<float>(), sc.p, sc.n, nullptr,
                                         qcodes.as<uint16_t>(), counts2.as<uint8_t>(),
                                         s_idx.as<int32_t>(), s_len.as<int32_t>()),
                  MP_OK);
    };
    decode_all(c.n);

    const float *W = nullptr, *mu = nullptr;
    const uint32_t *planes = nullptr;
    int32_t n_pad = 0;
    EXPECT_ST(mp_index_views(idx, &W, &mu, &planes, &n_pad), MP_OK);
    EXPECT(n_pad % 512 == 0 && n_pad >= c.n && n_pad - c.n < 512);
    const float *wx = nullptr, *r = nullptr;
    EXPECT_ST(mp_index_lift_views(idx, &wx, &r), (c.flags & MP_INDEX_MIPS) ? MP_OK : MP_E_ARG);

    if (c.grow_to > c.n) {
        // grow in two steps: to the middle, then to grow_to (tables are dropped)
        const int32_t mid = c.n + (c.grow_to - c.n) / 2;
        mp_kv_view km = keys.prefix(mid);
        EXPECT_ST(mp_index_append(idx, &km, nullptr), MP_OK);
        kv = keys.prefix(c.grow_to);
        vv = vals.prefix(c.grow_to);
        // the second step appended by a decode (at most kAppendMax new keys
        // with K > 0: their codes written by the query-encode launch; else
        // the two calls).  A refused call leaves the index as it was.
        {
            mp_kv_view kbad = kv;
            kbad.dtype = c.dtype == MP_BF16 ? MP_F32 : MP_BF16;
            EXPECT_ST(mp_decode_attn_append(q.as<float>(), H_q, idx, &kbad, &vv, 4, 64, 0.0f,
                                            out.as<float>(), w.p, ws, nullptr),
                      MP_E_DTYPE);
            EXPECT_ST(mp_decode_attn_append(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                            out.as<float>(), w.p, 64, nullptr),
                      MP_E_WORKSPACE);
            EXPECT_ST(mp_decode_attn_append(q.as<float>(), H_q + 1, idx, &kv, &vv, 4, 64, 0.0f,
                                            out.as<float>(), w.p, ws, nullptr),
                      MP_E_SHAPE);
            mp_kv_view vm = vals.prefix(mid);
            Buf sc(mp_decode_scratch_bytes(idx, H_q));
            EXPECT_ST(mp_decode_attn(q.as<float>(), H_q, idx, &km, &vm, 4, 64, 0.0f,
                                     out.as<float>(), sc.p, sc.n, nullptr),
                      MP_OK);   // still mid keys
            EXPECT_ST(mp_decode_attn_append(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f,
                                            out.as<float>(), sc.p, sc.n, nullptr),
                      MP_OK);
            EXPECT_ST(mp_decode_attn(q.as<float>(), H_q, idx, &km, &vm, 4, 64, 0.0f,
                                     out.as<float>(), sc.p, sc.n, nullptr),
                      MP_E_SHAPE);   // grown
        }
        EXPECT_ST(mp_index_append(idx, &kv, nullptr), MP_OK);   // nothing more to add
        EXPECT_ST(mp_tables_views(idx, nullptr, nullptr), MP_E_ARG);
        EXPECT_ST(mp_decode_attn_append(q.as<float>(), H_q, idx, &km, &km, 4, 64, 0.0f,
                                        out.as<float>(), w.p, ws, nullptr),
                  MP_E_SHAPE);   // fewer keys
        EXPECT_ST(mp_index_append(idx, &km, nullptr), MP_E_SHAPE);   // fewer keys
        EXPECT_ST(mp_index_views(idx, nullptr, nullptr, nullptr, &n_pad), MP_OK);
        EXPECT(n_pad >= c.grow_to && n_pad - c.grow_to < 512);
        decode_all(c.grow_to);
    }
    mp_index_destroy(idx);
    // the handle is dead: refused without touching freed memory
    EXPECT_ST(mp_decode_attn(q.as<float>(), H_q, idx, &kv, &vv, 4, 64, 0.0f, out.as<float>(),
                             w.p, ws, nullptr),
              MP_E_HANDLE);
    EXPECT(mp_decode_scratch_bytes(idx, H_q) == 0);
    mp_index_destroy(idx);   // a second destroy is a no-op
}

// ------------------------------------------------------------ error paths ----

static void error_paths()
{
    printf("case error_paths\n");
    fflush(stdout);
    KV keys(MP_BF16, 1, 2, 1000), vals(MP_BF16, 1, 2, 1000);
    const size_t ws = mp_index_workspace_bytes(1, 2, 1000, 128, 8, 20);
    Buf w(ws);
    mp_index *idx = nullptr;

    // size queries
    EXPECT(mp_index_workspace_bytes(1, 2, 1000, 64, 8, 20) == 0);
    EXPECT(mp_index_workspace_bytes(0, 2, 1000, 128, 8, 20) == 0);
    EXPECT(mp_index_workspace_bytes(1, 2, 0, 128, 8, 20) == 0);
    EXPECT(mp_index_workspace_bytes(1, 2, 1000, 128, 17, 20) == 0);
    EXPECT(mp_index_workspace_bytes(1, 2, 1000, 128, -1, 20) == 0);
    EXPECT(mp_index_workspace_bytes(1, 2, 1000, 128, 8, 1) == 0);
    EXPECT(mp_index_workspace_bytes(1, 2, 1000, 128, 8, 256) == 0);
    EXPECT(mp_index_workspace_bytes(65535, 1, 1, 128, 1, 2) > 0);
    EXPECT(mp_index_workspace_bytes(65536, 1, 1, 128, 1, 2) == 0);
    EXPECT(mp_index_workspace_bytes(1, 1, MP_MAX_KEYS, 128, 16, 255) > 0);
    EXPECT(mp_index_workspace_bytes(1, 1, MP_MAX_KEYS + 1, 128, 16, 255) == 0);
    EXPECT(mp_index_workspace_bytes(1, 1, 0x7FFFFFFF, 128, 10, 150) == 0);
    EXPECT(mp_index_workspace_bytes_ex(1, 2, 1000, 128, 8, 20, 2) == 0);

    // build: views
    mp_kv_view v = keys.view;
    EXPECT_ST(mp_build_index(nullptr, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, nullptr), MP_E_ARG);
    v.data = nullptr;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    v = keys.view;
    v.dtype = 7;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_DTYPE);
    v = keys.view;
    v.d = 64;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.n = 0;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.n = MP_MAX_KEYS + 1;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.stride_n = 100;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.stride_h = -128;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.data = keys.buf.as<char>() + 2;
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    v.stride_n = 132;   // 264-byte rows are not 16-byte aligned
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_SHAPE);
    v = keys.view;
    // build: parameters and workspace
    EXPECT_ST(mp_build_index(&v, 17, 20, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index(&v, -1, 20, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index(&v, 8, 1, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index(&v, 8, 256, 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index_ex(&v, 8, 20, 1, 1000, 8, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index_cap(&v, 8, 20, 1, 999, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index_cap(&v, 8, 20, 1, MP_MAX_KEYS + 1, w.p, ws, nullptr, &idx), MP_E_ARG);
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, nullptr, ws, nullptr, &idx), MP_E_WORKSPACE);
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.as<char>() + 16, ws - 16, nullptr, &idx),
              MP_E_WORKSPACE);
    EXPECT(idx == nullptr);

    // launch failures: the handle is not returned and not leaked
    mp_debug_fail_launches(0, 1);
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_HIP);
    EXPECT(idx == nullptr);
    mp_debug_fail_launches(2, 1);
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_E_HIP);
    EXPECT(idx == nullptr);
    mp_debug_fail_launches(0, 0);

    // a live index for the decode checks
    EXPECT_ST(mp_build_index(&v, 8, 20, 1, w.p, ws, nullptr, &idx), MP_OK);
    if (!idx) return;
    const int32_t H_q = 8;
    Buf q(H_q * 128 * 4), out(H_q * 128 * 4);
    const size_t sb = mp_decode_scratch_bytes(idx, H_q);
    Buf sc(sb);
    float *qf = q.as<float>(), *of = out.as<float>();
    mp_kv_view k = keys.view, vl = vals.view;
    auto dec = [&](const float *qq, int32_t hq, const mp_index *ix, const mp_kv_view *kk,
                   const mp_kv_view *vv, int32_t ns, int32_t nl, float scl, float *oo, void *s,
                   size_t sn) {
        return mp_decode_attn(qq, hq, ix, kk, vv, ns, nl, scl, oo, s, sn, nullptr);
    };
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_OK);
    EXPECT_ST(dec(qf, H_q, nullptr, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_HANDLE);
    EXPECT_ST(dec(qf, H_q, reinterpret_cast<const mp_index *>(w.p), &k, &vl, 4, 64, 0.0f, of,
                  sc.p, sc.n),
              MP_E_HANDLE);   // never dereferenced
    EXPECT_ST(dec(nullptr, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, nullptr, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf + 1, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, 0, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);
    EXPECT_ST(dec(qf, 7, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);
    EXPECT_ST(dec(qf, 6, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);   // G = 3
    EXPECT_ST(dec(qf, 32, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);  // G = 16
    EXPECT_ST(dec(qf, H_q, idx, nullptr, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, nullptr, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    mp_kv_view k2 = k;
    k2.n = 999;
    EXPECT_ST(dec(qf, H_q, idx, &k2, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);
    k2 = k;
    k2.H = 1;
    EXPECT_ST(dec(qf, H_q, idx, &k2, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_SHAPE);
    k2 = vl;
    k2.dtype = MP_F32;
    EXPECT_ST(dec(qf, H_q, idx, &k, &k2, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_DTYPE);
    k2 = k;
    k2.dtype = MP_F32;
    EXPECT_ST(dec(qf, H_q, idx, &k2, &k2, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_DTYPE);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, -1, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, -1, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, -1.0f, of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, __builtin_nanf(""), of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, __builtin_inff(), of, sc.p, sc.n), MP_E_ARG);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, nullptr, sc.n), MP_E_WORKSPACE);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.as<char>() + 128, sc.n - 128),
              MP_E_WORKSPACE);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, 64), MP_E_WORKSPACE);
    EXPECT(mp_decode_scratch_bytes(idx, 7) == 0 && mp_decode_scratch_bytes(idx, 0) == 0);
    EXPECT(mp::decode_scratch_needed(idx, 7) == -1);

    // the index lives on device 0: another current device is refused
    g_device = 1;
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_ARG);
    g_device = 0;

    // decode launch failure leaves the index usable
    mp_debug_fail_launches(0, 1);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_E_HIP);
    EXPECT_ST(dec(qf, H_q, idx, &k, &vl, 4, 64, 0.0f, of, sc.p, sc.n), MP_OK);

    // tables: failed build leaves no tables behind
    const size_t tw = mp_tables_workspace_bytes(idx);
    EXPECT(tw > 0);
    {
        Buf t(tw);
        EXPECT_ST(mp_build_tables(nullptr, t.p, tw, nullptr), MP_E_HANDLE);
        EXPECT_ST(mp_build_tables(idx, nullptr, tw, nullptr), MP_E_WORKSPACE);
        EXPECT_ST(mp_build_tables(idx, t.as<char>() + 64, tw - 64, nullptr), MP_E_WORKSPACE);
        g_device = 1;
        EXPECT_ST(mp_build_tables(idx, t.p, tw, nullptr), MP_E_ARG);
        g_device = 0;
        mp_debug_fail_launches(0, 1);
        EXPECT_ST(mp_build_tables(idx, t.p, tw, nullptr), MP_E_HIP);
        EXPECT_ST(mp_tables_views(idx, nullptr, nullptr), MP_E_ARG);
    }

    // append
    KV more(MP_BF16, 1, 2, 1500);
    mp_kv_view a = more.view;
    EXPECT_ST(mp_index_append(idx, &a, nullptr), MP_E_SHAPE);   // beyond capacity
    a = more.prefix(999);
    EXPECT_ST(mp_index_append(idx, &a, nullptr), MP_E_SHAPE);
    a = more.prefix(1000);
    EXPECT_ST(mp_index_append(idx, &a, nullptr), MP_OK);        // no new keys: nothing to do
    a.H = 1;
    EXPECT_ST(mp_index_append(idx, &a, nullptr), MP_E_SHAPE);
    a = more.prefix(1000);
    a.dtype = MP_F32;
    EXPECT_ST(mp_index_append(idx, &a, nullptr), MP_E_DTYPE);
    EXPECT_ST(mp_index_append(nullptr, &a, nullptr), MP_E_HANDLE);
    // append and decode in one call: refused before any launch
    a = more.prefix(999);
    EXPECT_ST(mp_decode_attn_append(nullptr, 4, idx, &a, &a, 4, 64, 0.0f, nullptr, nullptr, 0,
                                    nullptr),
              MP_E_SHAPE);   // fewer keys
    a = more.prefix(1001);
    EXPECT_ST(mp_decode_attn_append(nullptr, 4, idx, &a, &a, 4, 64, 0.0f, nullptr, nullptr, 0,
                                    nullptr),
              MP_E_SHAPE);   // beyond capacity
    a = more.view;
    EXPECT_ST(mp_decode_attn_append(nullptr, 4, idx, &a, &a, 4, 64, 0.0f, nullptr, nullptr, 0,
                                    nullptr),
              MP_E_SHAPE);   // beyond capacity, more than one launch's worth of keys
    EXPECT_ST(mp_decode_attn_append(nullptr, 4, nullptr, &a, &a, 4, 64, 0.0f, nullptr, nullptr,
                                    0, nullptr),
              MP_E_HANDLE);
    mp_index_destroy(idx);

    // a lifted index does not grow
    const size_t wsx = mp_index_workspace_bytes_ex(1, 2, 1000, 128, 8, 20, MP_INDEX_MIPS);
    Buf wx(wsx);
    EXPECT_ST(mp_build_index_ex(&v, 8, 20, 1, 1000, MP_INDEX_MIPS, wx.p, wsx, nullptr, &idx),
              MP_OK);
    if (idx) {
        EXPECT_ST(mp_index_append(idx, &v, nullptr), MP_E_ARG);
        mp_kv_view a1 = more.prefix(1001);
        EXPECT_ST(mp_decode_attn_append(nullptr, 4, idx, &a1, &a1, 4, 64, 0.0f, nullptr, nullptr,
                                        0, nullptr),
                  MP_E_ARG);
        mp_index_destroy(idx);
    }

    // tables refused for K > 12 and for n past the LDS bound at L = 255
    {
        const size_t w13 = mp_index_workspace_bytes(1, 2, 1000, 128, 13, 20);
        Buf b13(w13);
        EXPECT_ST(mp_build_index(&v, 13, 20, 1, b13.p, w13, nullptr, &idx), MP_OK);
        if (idx) {
            EXPECT(mp_tables_workspace_bytes(idx) == 0);
            EXPECT(mp_decode_tables_scratch_bytes(idx, 8) == 0);
            EXPECT_ST(mp_build_tables(idx, b13.p, w13, nullptr), MP_E_SHAPE);
            mp_index_destroy(idx);
        }
        // n = 1256 chunks is the largest at L = 255; checked on the layout alone
        mp::IndexLayout y = mp::index_layout(1, 1, 1256 * 512, 10, 255);
        EXPECT(mp::tables_unsupported(y) == nullptr);
        y = mp::index_layout(1, 1, 1256 * 512 + 1, 10, 255);
        EXPECT(mp::tables_unsupported(y) != nullptr);
    }

    // status strings
    for (int s = 0; s <= 6; ++s) EXPECT(strncmp(mp_status_str(mp_status(s)), "MP_", 3) == 0);
    EXPECT(strcmp(mp_status_str(mp_status(7)), "unknown mp_status") == 0);

    // long messages are cut to the buffer, terminated
    std::vector<char> longname(2000, 'x');
    longname.back() = 0;
    mp::fail(MP_E_ARG, "%s", longname.data());
    EXPECT(strlen(mp_last_error()) == 511);
}

// -------------------------------------------------------------- threads ----

// Builds, decodes and destroys indexes from several threads at once: the
// handle registry and the per-thread error text are shared state.
static void threads()
{
    printf("case threads\n");
    fflush(stdout);
    constexpr int kThreads = 8, kIters = 40;
    std::vector<std::thread> ts;
    std::atomic<int> bad{0};
    for (int t = 0; t < kThreads; ++t)
        ts.emplace_back([t, &bad] {
            KV keys(MP_BF16, 1, 1, 300 + 64 * t), vals(MP_BF16, 1, 1, 300 + 64 * t);
            const size_t ws = mp_index_workspace_bytes(1, 1, keys.view.n, 128, 6, 12);
            Buf w(ws), q(4 * 128 * 4), out(4 * 128 * 4);
            for (int it = 0; it < kIters; ++it) {
                mp_index *idx = nullptr;
                if (mp_build_index(&keys.view, 6, 12, it, w.p, ws, nullptr, &idx) != MP_OK) {
                    ++bad;
                    continue;
                }
                const size_t sb = mp_decode_scratch_bytes(idx, 4);
                Buf sc(sb);
                if (mp_decode_attn(q.as<float>(), 4, idx, &keys.view, &vals.view, 4, 16, 0.0f,
                                   out.as<float>(), sc.p, sc.n, nullptr) != MP_OK)
                    ++bad;
                // a refused call sets this thread's text only
                if (mp_decode_attn(q.as<float>(), 3, idx, &keys.view, &vals.view, 4, 16, 0.0f,
                                   out.as<float>(), sc.p, sc.n, nullptr) != MP_E_SHAPE ||
                    strstr(mp_last_error(), "H_q/H_kv = 3") == nullptr)
                    ++bad;
                mp_index_destroy(idx);
                if (mp_decode_scratch_bytes(idx, 4) != 0) ++bad;
            }
        });
    for (auto &th : ts) th.join();
    EXPECT(bad.load() == 0);
}

// ----------------------------------------------------------------- main ----

int main(int argc, char **argv)
{
    const char *what = argc > 1 ? argv[1] : "all";
    const bool all = strcmp(what, "all") == 0;
    if (all) {
        error_paths();
        const Case cases[] = {
            // name, dtype, B, H_kv, n, K, L, G, n_cap, flags, grow_to, pitch
            {"bf16_gqa4_ragged", MP_BF16, 1, 2, 1673, 10, 150, 4, 0, 0, 0, 128},
            {"fp32_batch2_gqa8", MP_F32, 2, 2, 1100, 9, 120, 8, 0, 0, 0, 128},
            {"one_key", MP_BF16, 1, 1, 1, 4, 16, 1, 0, 0, 0, 128},
            {"one_chunk_exact", MP_BF16, 1, 3, 512, 6, 40, 2, 0, 0, 0, 128},
            {"chunk_plus_one", MP_BF16, 1, 1, 513, 6, 40, 4, 0, 0, 0, 128},
            {"K0", MP_BF16, 1, 2, 1300, 0, 8, 4, 0, 0, 0, 128},
            {"K16_L255_no_tables", MP_BF16, 1, 1, 700, 16, 255, 2, 0, 0, 0, 128},
            {"K12_L255", MP_BF16, 1, 1, 600, 12, 255, 4, 0, 0, 0, 128},
            {"strided_rows", MP_BF16, 2, 2, 900, 8, 30, 2, 0, 0, 0, 192},
            {"fp32_strided", MP_F32, 1, 2, 777, 8, 30, 4, 0, 0, 0, 132},
            {"mips", MP_BF16, 1, 2, 2000, 10, 60, 4, 0, MP_INDEX_MIPS, 0, 128},
            {"grow", MP_BF16, 1, 2, 1000, 10, 60, 4, 3000, 0, 2900, 128},
            {"grow_K0", MP_BF16, 1, 1, 257, 0, 10, 8, 1200, 0, 1100, 128},
            {"grow_small", MP_BF16, 1, 2, 1000, 10, 60, 4, 1100, 0, 1003, 128},
            {"grow_small_across_chunk", MP_F32, 2, 1, 510, 9, 40, 2, 600, 0, 514, 128},
            {"grow_by_64_then_65", MP_BF16, 1, 2, 700, 10, 30, 4, 900, 0, 829, 128},
            {"llama8b_like_20k", MP_BF16, 1, 8, 20000, 10, 150, 4, 0, 0, 0, 128},
        };
        for (const Case &c : cases) run_case(c);
    }
    if (all || strcmp(what, "threads") == 0) threads();
    if (g_failed) {
        fprintf(stderr, "%d check(s) failed\n", g_failed);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
