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

// Gather form: output row m quantises row rows[m] of x ([src_rows, ldx]).
hipError_t launch_quant_act_gather(const uint16_t *x, int64_t src_rows, int64_t ldx, const int32_t *rows,
                                   int64_t M, int64_t K, int8_t *xq, float *xs, hipStream_t stream);

// Per-channel form (blocks of 1 x K): xs [M, 1], ws [N, 1], K <= 2^17.
hipError_t launch_gemm_per_channel(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                                   const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream);
// Per-token activation quantisation (one group of K per row).
hipError_t launch_quant_act_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                                      float *xs, hipStream_t stream);

// Offline block quantisation of a bf16 weight (128 x 128 blocks).
hipError_t launch_quant_weight(const uint16_t *w, int64_t N, int64_t K, int64_t ldw, int8_t *wq, float *ws,
                               hipStream_t stream);

// MoE steps around the grouped GEMM (E <= 1024, k <= 8).
hipError_t launch_moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renorm,
                            int32_t *ids, float *weights, int32_t *sorted_token, int32_t *offsets,
                            int32_t *row_of, hipStream_t stream);
hipError_t launch_silu_mul_quant(const uint16_t *h, int64_t R, int64_t I, int8_t *aq, float *as,
                                 uint16_t *a_out, hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t *y2, int64_t R, const int32_t *row_of, const float *w,
                              int64_t T, int32_t k, int64_t H, uint16_t *out, hipStream_t stream);

// Split K on a caller workspace for grids of few tiles (splits 1: no split).
int32_t splitk_splits(int64_t M, int64_t N, int64_t K);
int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_ws(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                          const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K, float *workspace,
                          int64_t workspace_bytes, hipStream_t stream);

hipError_t launch_gemm(GemmPath path, const int8_t *xq, const float *xs, const int8_t *w,
                       const float *ws, const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream);

// Host-side helpers of the C ABI layer (abi.cpp): the thread-local error
// message, the linear's argument checks and its two launches.
int32_t fail_status(int32_t status, const char *fmt, ...);
int32_t call_status(const char *fn, hipError_t e);
int32_t check_linear_args(const char *fn, const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                          const uint16_t *bias, const uint16_t *y, int64_t M, int64_t N, int64_t K,
                          int32_t block_n, int32_t block_k);
hipError_t launch_linear(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const uint16_t *bias,
                         uint16_t *y, int64_t M, int64_t N, int64_t K, int32_t block_n, int32_t block_k,
                         int8_t *xq, float *xs, hipStream_t st);

int64_t moe_gemm_workspace_bytes(int64_t R, int64_t N, int64_t K, int32_t E);
hipError_t launch_moe_gemm_ws(const int8_t *xq, const float *xs, const int32_t *offsets, const int8_t *w,
                              const float *ws, uint16_t *y, int64_t R, int64_t N, int64_t K, int32_t E,
                              float *workspace, int64_t workspace_bytes, hipStream_t stream);
hipError_t launch_moe_gemm_silu_quant(const int8_t *xq, const float *xs, const int32_t *offsets, const int8_t *w13,
                                      const float *ws13, int8_t *aq, float *as, int64_t R, int64_t I, int64_t K,
                                      int32_t E, hipStream_t stream);
hipError_t launch_moe_gemm(GemmPath path, const int8_t *xq, const float *xs, const int32_t *offsets,
                           const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N,
                           int64_t K, int32_t E, hipStream_t stream);

}  // namespace bi8
