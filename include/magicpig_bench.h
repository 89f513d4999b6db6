/*
 * magicpig_bench.h -- measurement aids of libmagicpig, apart from the decode
 * path: entry points that time the dominant kernel of a decode step, and a
 * plain streaming read that gives the device's HBM read rate.  The benchmark
 * uses them; an application needs only magicpig.h.
 */
#ifndef MAGICPIG_BENCH_H
#define MAGICPIG_BENCH_H

#include "magicpig.h"

#ifdef __cplusplus
extern "C" {
#endif

/* mp_decode_attn that also stamps two caller-created hipEvent_t (passed as
 * void*, either may be NULL) with the start and the end of the fused
 * collision-scan + gather kernel (they are handed to the kernel's launch, so
 * no other command sits between them and the kernel), so the caller can time
 * that kernel on its own.  Used by the benchmark; the output is that of
 * mp_decode_attn. */
mp_status mp_decode_attn_timed(const float *q, int32_t H_q, const mp_index *idx,
                               const mp_kv_view *k, const mp_kv_view *v,
                               int32_t n_sink, int32_t n_local, float scale, float *out,
                               void *scratch, size_t scratch_bytes, void *stream,
                               void *ev_scan_begin, void *ev_scan_end);

/* mp_decode_attn_tables that also stamps two caller-created hipEvent_t with
 * the start and end of the gather kernel (as mp_decode_attn_timed does for
 * the scan kernel).  Used by the benchmark. */
mp_status mp_decode_attn_tables_timed(const float *q, int32_t H_q, const mp_index *idx,
                                      const mp_kv_view *k, const mp_kv_view *v, int32_t n_sink,
                                      int32_t n_local, float scale, float *out, void *scratch,
                                      size_t scratch_bytes, void *stream, void *ev_gather_begin,
                                      void *ev_gather_end);

/* A plain streaming read of `bytes` (16-byte aligned device memory) by
 * `blocks` workgroups of 256 threads: the HBM read rate of this device, the
 * reference the benchmark reports beside its kernels' rates.  `sink` is a
 * device word that is practically never written.  MP_E_ARG on bad arguments. */
mp_status mp_stream_read(const void *data, int64_t bytes, uint32_t *sink, int32_t blocks,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAGICPIG_BENCH_H */
