// Host-side launchers of the block-wise INT8 kernels.  Arguments have been
// validated by the C ABI layer (abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi8 {

// Kernel paths for the dense GEMM, chosen by shape in select_gemm_path().
enum class GemmPath : int { kSkinny = 0, kTiledLarge = 1, kTiledSmall = 2 };

GemmPath select_gemm_path(int64_t M, int64_t N, int64_t K);

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                            float *xs, hipStream_t stream);

hipError_t launch_gemm(GemmPath path, const int8_t *xq, const float *xs, const int8_t *w,
                       const float *ws, const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream);

hipError_t launch_moe_gemm(const int8_t *xq, const float *xs, const int32_t *offsets,
                           const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N,
                           int64_t K, int32_t E, hipStream_t stream);

}  // namespace bi8
