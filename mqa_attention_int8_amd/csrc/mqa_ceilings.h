/* mqa_ceilings.h - measurement kernels for the benchmark (libmqa_ceilings.so).
 *
 * Not part of the attention library. They give the achievable ceilings that
 * the attention kernels are compared with: one-pass streaming from HBM and
 * dense bf16 matrix-core throughput on this GPU. Pointers are device
 * pointers; calls are asynchronous on `stream` (a hipStream_t, NULL for the
 * default stream). Return codes: 0 ok, 1 a NULL pointer, 2 a size out of
 * range, 6 the launch failed.
 */
#ifndef MQA_CEILINGS_H
#define MQA_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16; src 16-byte aligned) once with `blocks`
 * work-groups of 256 threads; partial[blocks] receives each work-group's
 * 32-bit wrapping sum of the 32-bit words it read (their total is the sum of
 * every word of the buffer, mod 2^32). */
int mqa_ceiling_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* partial, void* stream);

/* `blocks` work-groups of 8 waves; every wave issues iters x 8 bf16 MFMAs of
 * 16 x 16 x 32. sink: fp32 [blocks * 512], one value per thread. */
int mqa_ceiling_mfma_bf16(int32_t blocks, int32_t iters, float* sink, void* stream);

/* Flops (2 per multiply-add) of one mqa_ceiling_mfma_bf16 call. */
double mqa_ceiling_mfma_bf16_flops(int32_t blocks, int32_t iters);

#ifdef __cplusplus
}
#endif

#endif /* MQA_CEILINGS_H */
