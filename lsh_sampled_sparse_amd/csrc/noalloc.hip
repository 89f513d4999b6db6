// noalloc.hip -- mp_decode_attn_noalloc: the decode step with its scratch in
// a static device array of the library, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, from the module's load until the
// process ends.  In host code the name `scratch` is only a host-side stand-in;
// its device address on each GPU comes from hipGetSymbolAddress, taken once
// per device (with that device current) and kept, and only that address is
// handed to kernels.  Every call on a GPU uses that GPU's one array, so calls
// that overlap on one GPU (other streams, other threads) race: order them on
// one stream.  The decode writes every scratch word before it reads it in the
// same call (query codes, norms, partial records), so nothing in the array has
// to start at zero; it keeps whatever the last call left.
#include "mp_internal.h"

namespace mp {
namespace {

static __device__ __align__(256) unsigned char scratch[MP_NOALLOC_SCRATCH_BYTES];

PerDevice g_scratch_once;
void *g_scratch_ptr[PerDevice::kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the
// device's first call and kept.
hipError_t static_scratch_ptr(void **p)
{
    hipError_t e = g_scratch_once.once([](int dev) {
        void *ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (r == hipSuccess) g_scratch_ptr[dev] = ptr;
        return r;
    });
    if (e != hipSuccess) return e;
    int dev = -1;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    *p = g_scratch_ptr[dev];
    return *p ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace
}  // namespace mp

using namespace mp;

extern "C" mp_status mp_decode_attn_noalloc(const float *q, int32_t H_q, const mp_index *idx,
                                            const mp_kv_view *k, const mp_kv_view *v,
                                            int32_t n_sink, int32_t n_local, float scale,
                                            float *out, void *stream)
{
    const int64_t need = decode_scratch_needed(idx, H_q);
    if (need > int64_t(MP_NOALLOC_SCRATCH_BYTES))
        return fail(MP_E_WORKSPACE,
                    "this decode needs %lld bytes of scratch; the static scratch of "
                    "mp_decode_attn_noalloc holds %lld (MP_NOALLOC_SCRATCH_BYTES)",
                    (long long)need, (long long)MP_NOALLOC_SCRATCH_BYTES);
    void *p = nullptr;
    if (const hipError_t e = static_scratch_ptr(&p); e != hipSuccess)
        return fail(MP_E_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    // an invalid handle or H_q (need < 0) is reported by the common checks
    return decode_common(q, H_q, idx, k, v, n_sink, n_local, scale, out, p,
                         MP_NOALLOC_SCRATCH_BYTES, stream, false, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, false);
}
