// append_codes.h -- the codes of a few new keys, written into an index's bit
// planes in place: device code shared by the append launch of index_build.hip
// and the fused append-and-decode of decode.hip (page "MagicPIG: LSH Sampling
// for Efficient LLM Generation", system co-design: the sink and local tokens
// sit in a static cache beside the hashed keys, and a token leaving the local
// window joins the hashed keys).
#pragma once

#include "mp_internal.h"

namespace mp {

// Hyperplanes one block of an append covers: 64, each dotted by 4 lanes.
constexpr int kAppendRows = 64;

// Block (hyperplane block hb, unit u) of an append of keys [n0, n1) (at most
// kAppendMax new keys).  Thread t takes hyperplane r = 64 hb + t / 4 and the
// quarter t % 4 of the dims: the 4 lanes of a row read its 512 bytes as
// 64-byte pieces (float4 c of the quarter is float4 4c + t % 4 of the row),
// loaded before the block waits for its keys.  The new keys' centered rows
// x = k - mu (fp32, the build's mu) are staged in LDS sx; each lane dots its
// quarter of W_r with every new key, two shuffles add the quarters, and the
// sign bit goes into the word of plane row r (= l*K + b) that holds the key.
// Bits of the keys already indexed are kept: per word, one atomic AND clears
// the new keys' zero bits and one atomic OR sets their one bits.  The two
// touch disjoint bits, so their order does not matter, and nothing waits on
// them.  Every thread of the block calls it (it holds one barrier).
template <typename T>
__device__ __forceinline__ void append_codes_block(const T *__restrict__ keys, int64_t sb,
                                                   int64_t sh, int64_t sn, int32_t H, int32_t n0,
                                                   int32_t n1, int32_t nc_cap,
                                                   const float *__restrict__ mu,
                                                   const float *__restrict__ W, int32_t K,
                                                   int32_t L, uint32_t *__restrict__ planes, int u,
                                                   int hb, int t, float (*sx)[kD])
{
    const int nk = n1 - n0;
    const int r = hb * kAppendRows + (t >> 2), dq = t & 3;
    const bool live = r < K * L;
    float4 wr[8];
    {
        // a row past K*L reads row 0 (in bounds) and writes nothing
        const float4 *w4 = reinterpret_cast<const float4 *>(W + int64_t(live ? r : 0) * kD);
#pragma unroll
        for (int c = 0; c < 8; ++c) wr[c] = w4[4 * c + dq];
    }
    const T *kb = keys + (u / H) * sb + (u % H) * sh;
    const float *mu_u = mu + int64_t(u) * kD;
    for (int i = t; i < nk * kD; i += 256) {
        const int e = i / kD, d = i % kD;
        const T v = kb[int64_t(n0 + e) * sn + d];
        float f;
        if constexpr (sizeof(T) == 2) f = __uint_as_float(uint32_t(v) << 16);   // bf16
        else f = v;
        sx[e][d] = f - mu_u[d];
    }
    __syncthreads();
    uint32_t *row = planes + (int64_t(u) * nc_cap * (L * K) + r) * kWords;
    const int64_t chunk_stride = int64_t(L) * K * kWords;
    uint32_t *cur = nullptr, mask = 0u, val = 0u;
    for (int e = 0; e < nk; ++e) {
        const float4 *x4 = reinterpret_cast<const float4 *>(sx[e]);
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
            const float4 xa = x4[4 * c + dq], xb = x4[4 * c + 4 + dq];
            a0 = fmaf(wr[c].x, xa.x, a0);
            a0 = fmaf(wr[c].y, xa.y, a0);
            a0 = fmaf(wr[c].z, xa.z, a0);
            a0 = fmaf(wr[c].w, xa.w, a0);
            a1 = fmaf(wr[c + 1].x, xb.x, a1);
            a1 = fmaf(wr[c + 1].y, xb.y, a1);
            a1 = fmaf(wr[c + 1].z, xb.z, a1);
            a1 = fmaf(wr[c + 1].w, xb.w, a1);
        }
        float dot = a0 + a1;
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        if (dq != 0 || !live) continue;
        const int i = n0 + e;
        uint32_t *addr = row + (i / kChunk) * chunk_stride + (i % kChunk) / 32;
        if (addr != cur) {
            if (cur) {
                if (mask & ~val) atomicAnd(cur, ~(mask & ~val));
                if (val) atomicOr(cur, val);
            }
            cur = addr;
            mask = val = 0u;
        }
        mask |= 1u << (i & 31);
        if (dot > 0.0f) val |= 1u << (i & 31);
    }
    if (cur) {
        if (mask & ~val) atomicAnd(cur, ~(mask & ~val));
        if (val) atomicOr(cur, val);
    }
}

}  // namespace mp
