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

}  // namespace maxsim
