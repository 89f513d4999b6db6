// index_build.hip -- index build for MagicPIG decode on gfx950.
//
//   wgen          hyperplanes W ~ N(0,1), one shared matrix for all heads
//                 (page "MagicPIG: LSH Sampling for Efficient LLM Generation",
//                 system co-design item 2: one random projector serves every head)
//   mean          mu = mean of all n keys of each (sequence, KV head), fp64 sums
//                 (same page, method details: centering before hashing)
//   encode_keys   SimHash codes of x_i = k_i - mu on fp32 MFMA: bit j = [W_j.x_i > 0]
//                 (same page, background: SimHash sign(w^T x); method details:
//                 K x L vectors), stored as bit planes: per 512-key chunk and
//                 hyperplane j = l*K + b, 16 words whose bit i is bit b of the
//                 table-l code of key 32w + i.  A code costs its K bits.
#include "append_codes.h"
#include "mp_internal.h"

namespace mp {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- W
// SplitMix64 (Steele, Lea & Flood 2014): output number k of the generator
// started at `seed` is the finaliser applied to seed + k * golden-gamma.
__device__ __forceinline__ uint64_t splitmix_output(uint64_t seed, uint64_t k)
{
    uint64_t z = seed + k * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

// Normal number e of the stream: the cosine branch of the Box-Muller
// transform of the uniforms made from outputs 2e+1 and 2e+2.
__device__ __forceinline__ float normal_at(uint64_t seed, int64_t e)
{
    const uint64_t z1 = splitmix_output(seed, 2 * uint64_t(e) + 1);
    const uint64_t z2 = splitmix_output(seed, 2 * uint64_t(e) + 2);
    const double u1 = (double(z1 >> 11) + 1.0) * 0x1.0p-53;
    const double u2 = double(z2 >> 11) * 0x1.0p-53;
    return float(sqrt(-2.0 * log(u1)) * cos(2.0 * 3.141592653589793 * u2));
}

// Element e of W is normal number e of the stream.  Also writes the MFMA B-fragment
// copy: for column tile t (16 hyperplanes), lane = (j % 16) + 16 * (c / 32)
// and k-step s = c % 32 live at Wp[((t*8 + s/4)*64 + lane)*4 + s%4], so one
// float4 per lane per 4 k-steps is a contiguous 1 KB wave load.
__global__ __launch_bounds__(256) void wgen_kernel(uint64_t seed, int32_t R, int32_t R_pad,
                                                   float *__restrict__ W, float *__restrict__ Wp)
{
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= int64_t(R_pad) * kD) return;
    const int32_t j = int32_t(e / kD), c = int32_t(e % kD);
    const float g = j < R ? normal_at(seed, e) : 0.0f;
    W[e] = g;
    const int32_t t = j >> 4, lane = (j & 15) + 16 * (c >> 5), s = c & 31;
    Wp[((int64_t(t) * 8 + (s >> 2)) * 64 + lane) * 4 + (s & 3)] = g;
}

// The lift's extra coordinate of hyperplane j: normal number R*128 + j, the
// numbers right after those of W.
__global__ __launch_bounds__(256) void wgen_extra_kernel(uint64_t seed, int32_t R, int32_t R_pad,
                                                         float *__restrict__ wx)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < R_pad) wx[j] = j < R ? normal_at(seed, int64_t(R) * kD + j) : 0.0f;
}

// ---------------------------------------------------------------- loads
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// 8 consecutive elements of a row, as fp32.
template <typename T> struct Row8;
template <> struct Row8<float> {
    static __device__ __forceinline__ void load(const float *p, float (&o)[8])
    {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};
template <> struct Row8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[8])
    {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        o[0] = bf16_to_f32(a.x & 0xFFFFu); o[1] = bf16_to_f32(a.x >> 16);
        o[2] = bf16_to_f32(a.y & 0xFFFFu); o[3] = bf16_to_f32(a.y >> 16);
        o[4] = bf16_to_f32(a.z & 0xFFFFu); o[5] = bf16_to_f32(a.z >> 16);
        o[6] = bf16_to_f32(a.w & 0xFFFFu); o[7] = bf16_to_f32(a.w >> 16);
    }
};

// ---------------------------------------------------------------- mean
// Block (kMeanRows keys of one head): thread t sums dims 8*(t%16)..+7 over
// rows r0 + t/16 + 16k in fp64; the 16 row lanes are added in LDS in a fixed
// order, so the result does not depend on scheduling.
template <typename T>
__global__ __launch_bounds__(256) void mean_partial_kernel(const T *__restrict__ keys, int64_t sb,
                                                           int64_t sh, int64_t sn, int32_t H,
                                                           int32_t n, int32_t nmb,
                                                           double *__restrict__ mu_part)
{
    __shared__ double red[16][kD];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, dg = t & 15, ro = t >> 4;
    const int64_t r0 = int64_t(blockIdx.x) * kMeanRows;
    const int64_t r1 = r0 + kMeanRows < n ? r0 + kMeanRows : n;
    const T *base = keys + b * sb + h * sh + 8 * dg;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t i = r0 + ro; i < r1; i += 16) {
        float v[8];
        Row8<T>::load(base + i * sn, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += double(v[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) red[ro][8 * dg + k] = acc[k];
    __syncthreads();
    if (t < kD) {
        double s = 0.0;
        for (int r = 0; r < 16; ++r) s += red[r][t];
        mu_part[(int64_t(bh) * nmb + blockIdx.x) * kD + t] = s;
    }
}

__global__ __launch_bounds__(kD) void mean_final_kernel(const double *__restrict__ mu_part,
                                                        int32_t nmb, int32_t n,
                                                        float *__restrict__ mu,
                                                        double *__restrict__ mu64)
{
    const int bh = blockIdx.x, t = threadIdx.x;
    double s = 0.0;
    for (int c = 0; c < nmb; ++c) s += mu_part[(int64_t(bh) * nmb + c) * kD + t];
    mu[int64_t(bh) * kD + t] = float(s / double(n));
    if (mu64) mu64[int64_t(bh) * kD + t] = s / double(n);
}

// ---------------------------------------------------------------- lift norms
// |k_i - mu|^2 in fp64 for the kMeanRows keys of a block: a 16-lane group per
// key (lane = 8 dims), fp64 sums over the group by shuffles; the block's max
// goes to xmax.  The lift's extra coordinate sqrt(r^2 - |x|^2) cancels for
// keys near the largest norm, so these sums stay in fp64 throughout.
template <typename T>
__global__ __launch_bounds__(256) void lift_norm_kernel(const T *__restrict__ keys, int64_t sb,
                                                        int64_t sh, int64_t sn, int32_t H,
                                                        int32_t n, int32_t n_cap, int32_t nmb,
                                                        const double *__restrict__ mu64,
                                                        double *__restrict__ xx,
                                                        double *__restrict__ xmax)
{
    __shared__ double red[16];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, gi = t >> 4, li = t & 15;
    double m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = mu64[int64_t(bh) * kD + 8 * li + e];
    const T *base = keys + b * sb + h * sh + 8 * li;
    const int64_t r0 = int64_t(blockIdx.x) * kMeanRows;
    const int64_t r1 = r0 + kMeanRows < n ? r0 + kMeanRows : n;
    double best = 0.0;
    for (int64_t i = r0 + gi; i < r1; i += 16) {
        float v[8];
        Row8<T>::load(base + i * sn, v);
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double x = double(v[e]) - m[e];
            s = fma(x, x, s);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
        if (li == 0) xx[int64_t(bh) * n_cap + i] = s;
        best = s > best ? s : best;
    }
    if (li == 0) red[gi] = best;
    __syncthreads();
    if (t == 0) {
        double mx = 0.0;
        for (int g = 0; g < 16; ++g) mx = red[g] > mx ? red[g] : mx;
        xmax[int64_t(bh) * nmb + blockIdx.x] = mx;
    }
}

__global__ __launch_bounds__(64) void lift_final_kernel(const double *__restrict__ xmax,
                                                        int32_t nmb, double *__restrict__ r2,
                                                        float *__restrict__ rnorm)
{
    const int bh = blockIdx.x;
    if (threadIdx.x != 0) return;
    double mx = 0.0;
    for (int c = 0; c < nmb; ++c) mx = xmax[int64_t(bh) * nmb + c] > mx ? xmax[int64_t(bh) * nmb + c] : mx;
    r2[bh] = mx;
    rnorm[bh] = float(sqrt(mx));
}

// ---------------------------------------------------------------- encode
// One block = 4 waves = 256 consecutive keys of one head; wave w owns keys
// k0 = 256*(kb0 + blockIdx.x) + 64*w .. +63 as 4 tiles of 16.
//
// Contraction P[j][i] = sum_c W_j[c] x_i[c] on v_mfma_f32_16x16x4_f32
// (A 16x4, B 4x16, 16x16 fp32 accumulate), A = hyperplanes, B = keys.  The
// 128-long contraction is split in 32 k-steps; in k-step s, lane l feeds dim
// c = 32*(l/16) + s of hyperplane l%16 (A) and of key l%16 (B), so a lane
// reads 32 contiguous dims of one key row.  The result lane l holds
// hyperplanes 4*(l/16) + r of the tile, key l%16, so a ballot of register r
// gives the sign bits of 16 keys for each of 4 hyperplanes: a 16-bit piece of
// a plane word.  Pieces go to LDS ([hyperplane][key tile]) and leave as
// 32-key words once every hyperplane tile is done.
//
// W tiles (8 KB each, fragment order) are staged through a double-buffered LDS
// slot shared by the 4 waves.
template <typename T>
__global__ __launch_bounds__(256) void encode_keys_kernel(
    const T *__restrict__ keys, int64_t sb, int64_t sh, int64_t sn, int32_t H, int32_t n,
    int32_t nc_cap, const float *__restrict__ mu, const float *__restrict__ Wp, int32_t K,
    int32_t L, int32_t NT, uint32_t *__restrict__ planes, int32_t kb0,
    const float *__restrict__ wx, const double *__restrict__ xx, const double *__restrict__ r2,
    int32_t n_cap)
{
    extern __shared__ __align__(16) unsigned char smem[];
    float4 *wbuf = reinterpret_cast<float4 *>(smem);                       // [2][512] float4
    uint16_t *pieces = reinterpret_cast<uint16_t *>(smem + 2 * 512 * 16);  // [4][16 NT][4]

    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int il = lane & 15, g = lane >> 4;
    const int64_t k0 = int64_t(kb0 + blockIdx.x) * 256 + 64 * w;

    // B fragments: x = k - mu for 4 key tiles, dims 32g .. 32g+31.
    float a[4][32];
    {
        float m[32];
        const float *mp = mu + int64_t(bh) * kD + 32 * g;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(mp + 4 * q);
            m[4 * q] = v.x; m[4 * q + 1] = v.y; m[4 * q + 2] = v.z; m[4 * q + 3] = v.w;
        }
        const T *base = keys + b * sb + h * sh + 32 * g;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int64_t row = k0 + 16 * rt + il;
            if (row < n) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[8];
                    Row8<T>::load(base + row * sn + 8 * q, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[rt][8 * q + e] = v[e] - m[8 * q + e];
                }
            } else {
#pragma unroll
                for (int s = 0; s < 32; ++s) a[rt][s] = 0.0f;
            }
        }
    }

    // The lift (wx non-NULL): key row il of tile rt gains the coordinate
    // sqrt(r^2 - |x|^2) (0 for padding keys), projection j the term wx[j] times it.
    float lifted[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (wx) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int64_t row = k0 + 16 * rt + il;
            if (row < n) {
                const double d2 = r2[bh] - xx[int64_t(bh) * n_cap + row];
                lifted[rt] = float(d2 > 0.0 ? sqrt(d2) : 0.0);
            }
        }
    }

    const float4 *wp4 = reinterpret_cast<const float4 *>(Wp);
    float4 pre0 = wp4[t], pre1 = wp4[256 + t];
    wbuf[t] = pre0;
    wbuf[256 + t] = pre1;
    __syncthreads();

    uint16_t *mine = pieces + int64_t(w) * (16 * NT) * 4;
    for (int ct = 0; ct < NT; ++ct) {
        if (ct + 1 < NT) {
            pre0 = wp4[int64_t(ct + 1) * 512 + t];
            pre1 = wp4[int64_t(ct + 1) * 512 + 256 + t];
        }
        const float4 *cur = wbuf + (ct & 1) * 512;
        float bf[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float4 v = cur[q * 64 + lane];
            bf[4 * q] = v.x; bf[4 * q + 1] = v.y; bf[4 * q + 2] = v.z; bf[4 * q + 3] = v.w;
        }
        // lane l's results are hyperplanes 16 ct + 4 g + r
        const float4 wl = wx ? reinterpret_cast<const float4 *>(wx)[4 * ct + g]
                             : float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 32; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[s], a[rt][s], acc, 0, 0, 0);
            if (wx) {
                acc[0] = fmaf(wl.x, lifted[rt], acc[0]);
                acc[1] = fmaf(wl.y, lifted[rt], acc[1]);
                acc[2] = fmaf(wl.z, lifted[rt], acc[2]);
                acc[3] = fmaf(wl.w, lifted[rt], acc[3]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const unsigned long long m = __ballot(acc[r] > 0.0f);
                if (lane < 4)   // lane q: hyperplane 16 ct + 4 q + r, keys 16 rt .. +15
                    mine[(16 * ct + 4 * lane + r) * 4 + rt] = uint16_t((m >> (16 * lane)) & 0xFFFFu);
            }
        }
        if (ct + 1 < NT) {
            wbuf[((ct + 1) & 1) * 512 + t] = pre0;
            wbuf[((ct + 1) & 1) * 512 + 256 + t] = pre1;
        }
        __syncthreads();
    }

    // Plane words: item = (hyperplane j, half hf of the wave's 64 keys); the
    // two 16-bit pieces of a half are one 32-bit LDS word.
    const int chunk = int(k0 / kChunk), word0 = int(k0 % kChunk) / 32;
    uint32_t *pout = planes + (int64_t(bh) * nc_cap + chunk) * int64_t(K) * L * kWords + word0;
    const uint32_t *mine32 = reinterpret_cast<const uint32_t *>(mine);
    for (int it = lane; it < 2 * K * L; it += 64) {
        const int j = it >> 1, hf = it & 1;
        pout[int64_t(j) * kWords + hf] = mine32[2 * j + hf];
    }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int64_t count)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_wgen(uint64_t seed, int32_t R, int32_t R_pad, float *W, float *Wp, hipStream_t s)
{
    const int64_t total = int64_t(R_pad) * kD;
    return launch(wgen_kernel, dim3(ceil_div(total, 256)), dim3(256), 0, s, seed, R, R_pad, W, Wp);
}

hipError_t launch_mean(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                       int32_t nmb, double *mu_part, float *mu, double *mu64, hipStream_t s)
{
    const dim3 grid(nmb, B * H);
    hipError_t e =
        dtype == MP_BF16
            ? launch(mean_partial_kernel<uint16_t>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t *>(keys.data), keys.sb, keys.sh, keys.sn, H, n,
                     nmb, mu_part)
            : launch(mean_partial_kernel<float>, grid, dim3(256), 0, s,
                     static_cast<const float *>(keys.data), keys.sb, keys.sh, keys.sn, H, n, nmb,
                     mu_part);
    if (e != hipSuccess) return e;
    return launch(mean_final_kernel, dim3(B * H), dim3(kD), 0, s, mu_part, nmb, n, mu, mu64);
}

hipError_t launch_wgen_extra(uint64_t seed, int32_t R, int32_t R_pad, float *wx, hipStream_t s)
{
    return launch(wgen_extra_kernel, dim3(ceil_div(R_pad, 256)), dim3(256), 0, s, seed, R, R_pad,
                  wx);
}

hipError_t launch_lift_norms(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                             int32_t n_cap, int32_t nmb, const double *mu64, double *xx,
                             double *xmax, double *r2, float *rnorm, hipStream_t s)
{
    const dim3 grid(nmb, B * H);
    hipError_t e =
        dtype == MP_BF16
            ? launch(lift_norm_kernel<uint16_t>, grid, dim3(256), 0, s,
                     static_cast<const uint16_t *>(keys.data), keys.sb, keys.sh, keys.sn, H, n,
                     n_cap, nmb, mu64, xx, xmax)
            : launch(lift_norm_kernel<float>, grid, dim3(256), 0, s,
                     static_cast<const float *>(keys.data), keys.sb, keys.sh, keys.sn, H, n, n_cap,
                     nmb, mu64, xx, xmax);
    if (e != hipSuccess) return e;
    return launch(lift_final_kernel, dim3(B * H), dim3(64), 0, s, xmax, nmb, r2, rnorm);
}

// Dynamic LDS of encode_keys_kernel: two 512-float key tiles and two W tiles
// of 16 NT hyperplanes x 4 floats x 4 k-steps; the largest is NT = 255
// (K L <= 16 x 255).
static size_t encode_keys_lds(int32_t NT) { return size_t(2) * 512 * 16 + size_t(4) * (16 * NT) * 4 * 2; }

hipError_t launch_encode_keys(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n,
                              int32_t nc_cap, const float *mu, const float *Wp, int32_t K,
                              int32_t L, int32_t R_pad, uint32_t *planes, int32_t kb0,
                              const float *wx, const double *xx, const double *r2, int32_t n_cap,
                              hipStream_t s)
{
    static PerDevice attr;
    hipError_t e = attr.once([](int) {
        const int most = int(encode_keys_lds(255));
        hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void *>(encode_keys_kernel<uint16_t>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, most);
        if (r == hipSuccess)
            r = hipFuncSetAttribute(reinterpret_cast<const void *>(encode_keys_kernel<float>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, most);
        return r;
    });
    if (e != hipSuccess) return e;
    const int32_t NT = R_pad / 16;
    const size_t shmem = encode_keys_lds(NT);
    // every 256-key block up to the end of the last chunk, so the padding
    // keys of the last chunk are written too (as zero rows)
    const int32_t nblocks = ceil_div(n, kChunk) * (kChunk / 256) - kb0;
    if (nblocks <= 0) return hipSuccess;
    const dim3 grid(nblocks, B * H);
    if (dtype == MP_BF16)
        return launch(encode_keys_kernel<uint16_t>, grid, dim3(256), shmem, s,
                      static_cast<const uint16_t *>(keys.data), keys.sb, keys.sh, keys.sn, H, n,
                      nc_cap, mu, Wp, K, L, NT, planes, kb0, wx, xx, r2, n_cap);
    return launch(encode_keys_kernel<float>, grid, dim3(256), shmem, s,
                  static_cast<const float *>(keys.data), keys.sb, keys.sh, keys.sn, H, n, nc_cap,
                  mu, Wp, K, L, NT, planes, kb0, wx, xx, r2, n_cap);
}

namespace {

// ---------------------------------------------------------------- small appends
// One block of append_codes_block (append_codes.h) per (hyperplane block,
// unit).  The work is that of the new keys alone, where re-encoding their
// 256-key block costs the MFMA work of 256 keys on one workgroup per unit.
template <typename T>
__global__ __launch_bounds__(256) void append_codes_kernel(const T *__restrict__ keys, int64_t sb,
                                                           int64_t sh, int64_t sn, int32_t H,
                                                           int32_t n0, int32_t n1, int32_t nc_cap,
                                                           const float *__restrict__ mu,
                                                           const float *__restrict__ W, int32_t K,
                                                           int32_t L, uint32_t *__restrict__ planes)
{
    __shared__ __align__(16) float sx[kAppendMax][kD];
    append_codes_block<T>(keys, sb, sh, sn, H, n0, n1, nc_cap, mu, W, K, L, planes, blockIdx.y,
                          blockIdx.x, threadIdx.x, sx);
}

}  // namespace

hipError_t launch_append_codes(const KVRows &keys, int32_t dtype, int32_t B, int32_t H, int32_t n0,
                               int32_t n1, int32_t nc_cap, const float *mu, const float *W,
                               int32_t K, int32_t L, uint32_t *planes, hipStream_t s)
{
    if (n1 <= n0 || K <= 0) return hipSuccess;
    if (n1 - n0 > kAppendMax) return hipErrorInvalidValue;
    const dim3 grid(ceil_div(int64_t(K) * L, kAppendRows), B * H);
    if (dtype == MP_BF16)
        return launch(append_codes_kernel<uint16_t>, grid, dim3(256), 0, s,
                      static_cast<const uint16_t *>(keys.data), keys.sb, keys.sh, keys.sn, H, n0, n1,
                      nc_cap, mu, W, K, L, planes);
    return launch(append_codes_kernel<float>, grid, dim3(256), 0, s,
                  static_cast<const float *>(keys.data), keys.sb, keys.sh, keys.sn, H, n0, n1, nc_cap,
                  mu, W, K, L, planes);
}

hipError_t launch_fill_u32(uint32_t *p, int64_t count, hipStream_t s)
{
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    return launch(fill_u32_kernel, dim3(uint32_t(blocks)), dim3(256), 0, s, p, count);
}

}  // namespace mp
