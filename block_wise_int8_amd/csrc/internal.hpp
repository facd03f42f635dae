// Host-side launchers of the block-wise INT8 kernels.  Arguments have been
// validated by the C ABI layer (abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi8 {

// GEMM kernels (the values are the BI8_GEMM_* variant ids of the C ABI).
enum class GemmPath : int { kAuto = 0, kSkinny = 1, kTile128x64 = 2, kTile256x128 = 3, kTile256x256 = 4 };

// Shape-based choice for the dense and the grouped GEMM (never kAuto).
GemmPath select_gemm_path(int64_t M, int64_t N, int64_t K);
GemmPath select_moe_gemm_path(int64_t R, int64_t N, int64_t K, int32_t E);

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                            float *xs, hipStream_t stream);

hipError_t launch_gemm(GemmPath path, const int8_t *xq, const float *xs, const int8_t *w,
                       const float *ws, const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream);

hipError_t launch_moe_gemm(GemmPath path, const int8_t *xq, const float *xs, const int32_t *offsets,
                           const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N,
                           int64_t K, int32_t E, hipStream_t stream);

}  // namespace bi8
