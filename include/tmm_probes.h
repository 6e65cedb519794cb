/*
 * Measurement kernels (libtmm_probes.so): the ceilings the library's
 * kernels are measured against on this chip, beside the published peaks.
 * They compute nothing of the product; bench.py times them with the same
 * launch shapes, sizes and timing method as the kernels they bound.
 *
 * Roofline model of the "GEMM to FlashAttention" page (roofline section:
 * attainable = min(peak, bandwidth x intensity)) and the batch-1 bound of
 * the CMU 15-418 Lecture 27 notes (section 7, question 1: a matrix-vector
 * product can go no faster than its weights stream in).  Both assume the
 * nameplate figures are reachable; these kernels measure what is:
 *
 *   tmmp_stream_read: the GEMV's access pattern without its arithmetic --
 *     one wave per row of `row_bytes` bytes, each lane issuing its 16-byte
 *     non-temporal loads of the row before using any, `waves_per_group`
 *     waves per workgroup; every byte of the rows x row_bytes array at `src`
 *     (device memory, 16-byte aligned, rows packed) is read once.
 *     row_bytes must be a positive multiple of 1024 and at most 65536;
 *     waves_per_group 1, 2, 4, 8 or 16; `sink` (device, 4 bytes) is written
 *     only under a data condition that does not occur for finite inputs, so
 *     the loads are kept.
 *
 *   tmmp_mfma_loop: the matrix cores alone -- `groups` workgroups of 8
 *     waves; each wave loads 24 16-byte operand fragments per lane from
 *     `operands` once, then issues `iters` rounds of matrix instructions on
 *     the accumulators of a 128x64 block (per wave), cycling through 4
 *     K-steps of fragments, so the operands change every instruction as in
 *     a GEMM.  shape 0: v_mfma_f32_32x32x16_bf16 (32 per round), shape 1:
 *     v_mfma_f32_16x16x32_bf16 (64 per round), shape 2: the fp8 (e4m3)
 *     32x32x64 (8 per round), shape 3: the fp8 16x16x128 (16 per round);
 *     1 Mi flop per round in every case (shapes 2, 3: iters a multiple of
 *     4; the fp8 operands are the same bytes read as e4m3).  `operands` holds operand_bytes >= max(16 MiB, groups x 192 KiB)
 *     of bf16 data (each thread reads its own 384 bytes; the caller's
 *     values: random data draws more power than zeros); `sink` (device)
 *     receives one float per thread, groups * 512 floats.
 *
 * Both return 0, TMM_ERR_DIM / TMM_ERR_NULL / TMM_ERR_ALIGN / TMM_ERR_ARG
 * for bad arguments (checked on the host before any HIP call) or
 * TMM_ERR_LAUNCH; they are asynchronous on `stream`.
 */
#ifndef TMM_PROBES_H
#define TMM_PROBES_H

#include <stdint.h>
#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

int tmmp_stream_read(const void *src, int64_t rows, int64_t row_bytes, int waves_per_group, int *sink,
                     hipStream_t stream);

int tmmp_mfma_loop(const void *operands, int64_t operand_bytes, int shape, int64_t groups, int64_t iters,
                   float *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
