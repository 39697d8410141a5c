/*
 * Measurement helpers shipped with libmaxsim (not part of the scoring path).
 *
 * maxsim_calib_read streams `bytes` from `src` with non-temporal 128-bit loads (each
 * wave reading whole 16 KiB blocks, `wgs_per_cu` workgroups of 4 waves per CU, <= 0 or
 * more than fit: as many as fit) and writes one word per workgroup to `sink` (so the
 * reads cannot be optimised away): its duration gives the achievable HBM read bandwidth
 * of the device, the ceiling a memory-bound scoring kernel can approach.
 * maxsim_calib_copy copies `bytes` from src to dst with 128-bit loads and stores:
 * a plain copy of known size, used to scale hardware traffic counters.
 *
 *   src, dst  device pointers, 16-byte aligned; bytes a multiple of 16
 *   sink      device fp32/uint32 buffer of at least 65536 words
 *   stream    hipStream_t (NULL = default stream)
 * Returns 0 or a negative maxsim_status code (include/maxsim.h).
 */
#ifndef MAXSIM_CALIB_H
#define MAXSIM_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int maxsim_calib_read(const void *src, size_t bytes, int wgs_per_cu, uint32_t *sink, void *stream);
/* Streams `bytes` of a fixed pattern into dst with 128-bit stores, each wave writing whole
 * 16 KiB blocks, `wgs_per_cu` workgroups of 4 waves per CU (<= 0 or more than fit: as many
 * as fit); contig != 0 gives each wave one contiguous range of blocks, else the blocks go
 * to the waves in turn: the achievable HBM write bandwidth, the ceiling of a kernel that
 * mostly writes (the backward's dD). dst 16-byte aligned, bytes % 16 == 0. */
int maxsim_calib_write(void *dst, size_t bytes, int wgs_per_cu, int contig, void *stream);
int maxsim_calib_copy(const void *src, void *dst, size_t bytes, void *stream);

/*
 * Matrix-core throughput: independent MFMA chains with no memory traffic, for the
 * achievable MFMA rate of the device. kind 0: 16x16x32 bf16, 1: 32x32x16 bf16,
 * 2: 16x16x64 int8, 3: 32x32x32 int8. waves_per_simd in [1, 8], iters >= 1.
 * *ops receives the FLOP (or integer op) count of the launch (host pointer);
 * sink is a device buffer of >= 65536 floats that the kernel does not write in practice.
 */
int maxsim_calib_mfma(int kind, int iters, int waves_per_simd, float *sink, double *ops,
                      void *stream);

/*
 * Vector-ALU throughput: 8 independent chains of fp32 fused multiply-adds per lane (one
 * non-packed VALU instruction each), waves_per_simd x 4 x CUs waves of `iters` rounds.
 * *ops receives the FLOP count (2 per lane and FMA).
 */
int maxsim_calib_valu(int iters, int waves_per_simd, float *sink, double *ops, void *stream);

/*
 * Matrix core and vector ALU side by side: per round 8 independent 16x16x64 int8 MFMA
 * chains and valu_per_mfma (0, 1, 2, 4 or 8) x 8 independent fp32 FMAs, with no data
 * flowing between them. Timed against valu_per_mfma = 0 and against maxsim_calib_valu it
 * shows how far the two units overlap. *ops receives the int8 MFMA integer-op count.
 */
int maxsim_calib_mix(int valu_per_mfma, int iters, int waves_per_simd, float *sink,
                     double *ops, void *stream);

/*
 * LDS read rate: one 1024-thread workgroup per CU with 128 KiB of LDS, every lane issuing
 * 16 x iters 16-byte reads. pattern 0: each wave reads 1 KiB of contiguous LDS per
 * instruction (conflict-free); pattern 1: the PQ lookup pattern (lane pairs share a token
 * and read the two halves of row (m, code) of a [16][256][8] fp32 table, codes random).
 * *bytes receives the LDS bytes read. sink: >= 65536 words, not written in practice.
 */
int maxsim_calib_lds(int pattern, int iters, uint32_t *sink, double *bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_CALIB_H */
