// Dense kernel dispatch: one translation unit per storage type instantiates the
// (chunks per d block, query blocks, pipeline depth, Q placement) variants.
#pragma once

#include "dense_kernel.hpp"
#include "host_common.hpp"

namespace maxsim {

int dense_dispatch_bf16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                        const DeviceInfo &di, hipStream_t st);
int dense_dispatch_fp16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                        const DeviceInfo &di, hipStream_t st);
int dense_dispatch_fp32(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                        const DeviceInfo &di, hipStream_t st);
// The same kernels writing per-token maxima and argmax (DenseArgs::tok_max / tok_arg).
int dense_argmax_dispatch_bf16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                               const DeviceInfo &di, hipStream_t st);
int dense_argmax_dispatch_fp16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                               const DeviceInfo &di, hipStream_t st);
int dense_argmax_dispatch_fp32(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                               const DeviceInfo &di, hipStream_t st);
// INT8 storage (DenseArgs::q_scale / d_scale), with per-token maxima and argmax where
// DenseArgs::tok_max is set; ksb = d / 64 in {1, 2, 4}, qb <= 4; defined in dense_i8.hip.
int dense_i8_run(int ksb, int qb, const DenseArgs &a, const DeviceInfo &di, hipStream_t st);
// Several short queries per pass (DenseArgs::n_q queries of q_len tokens in Q, out [n_q][B]):
// bf16 / fp16 rows of 128 or 256 bytes, at most DBATCH_MAX_BLOCKS 16-token query blocks
// (each query padded to whole blocks); defined in dense_batch.hip.
constexpr int DBATCH_MAX_BLOCKS = 16;
int dense_batch_blocks(int n_q, int q_len);
bool dense_batch_fits(int n_q, int q_len, int d, int dtype);
int dense_batch_run(const DenseArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st);

}  // namespace maxsim
