// probe.hip -- a plain streaming read, the HBM reference that the benchmark
// reports beside its kernels' rates (no part of the decode path).
#include "mp_internal.h"

namespace mp {
namespace {

// Grid-stride read of n16 16-byte words, four loads in flight per thread; the
// words are folded into one value that is written only if it takes a value
// no input of all-equal words produces, so the loads are kept but nothing is
// stored in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink)
{
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
               d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace mp

using namespace mp;

extern "C" mp_status mp_stream_read(const void *data, int64_t bytes, uint32_t *sink, int32_t blocks,
                                    void *stream)
{
    if (!data || !sink || bytes < 16 || blocks < 1 || (reinterpret_cast<uintptr_t>(data) & 15))
        return MP_E_ARG;
    return launch(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                  static_cast<const uint4 *>(data), bytes / 16, sink) == hipSuccess
               ? MP_OK
               : MP_E_HIP;
}
