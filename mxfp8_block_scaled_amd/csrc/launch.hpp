// Internal launchers behind the C ABI (one per kernel family).  Each assumes
// its arguments were validated by api.cpp and returns 0 or -7 (launch error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfp8 {

int launch_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq, void* s,
                        int64_t lds, hipStream_t stream);

// Same, written as packed operand tiles (common.hpp), rows padded to 128.
int launch_quantize_act_packed(const void* x, int64_t M, int64_t K, int64_t ldx, void* qp, void* sp,
                               hipStream_t stream);

int launch_pack_weight(const void* w, const void* ws, int64_t N, int64_t K, int64_t ldw, int64_t ldws,
                       void* wp, void* sp, hipStream_t stream);

int launch_unpack_weight(const void* wp, const void* sp, int64_t N, int64_t K, void* w, void* ws,
                         hipStream_t stream);

// Large-tile GEMM on packed activations (qp, sp: M rows) and the packed
// weight (wp, wsp: N rows).
int launch_gemm_tile(const void* qp, const void* sp, int64_t M, int64_t K, const void* wp, const void* wsp,
                     int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream);

// Skinny GEMM with the activation quantization fused in (M <= kSkinnyMaxM,
// K <= kSkinnyMaxK).
constexpr int64_t kSkinnyMaxM = 16;
constexpr int64_t kSkinnyMaxK = 8192;
int launch_gemm_skinny(const void* x, int64_t ldx, int64_t M, int64_t K, const void* wp, const void* sp,
                       int64_t N, const void* bias, void* y, int64_t ldy, hipStream_t stream);

}  // namespace mxfp8
