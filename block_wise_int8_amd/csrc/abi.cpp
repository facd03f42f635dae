// C ABI of the block-wise INT8 library: argument checks on the host, then
// one launch on the caller's stream.  See include/blockint8.h for the
// contract of each entry point.
//
// The checks mirror the configuration rules of the page "[SGLang] Block-wise
// INT8" (blog.secrett2633.cloud), section 1: weights arrive as int8 (the only
// weight type accepted here), the block has two dimensions (block_n,
// block_k), and only dynamic activation scales exist (there is no argument
// for a static one).  Everything is checked before any HIP call, so a bad
// call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/blockint8.h"
#include "internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int32_t ok() {
    g_last_error[0] = '\0';
    return BI8_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxRows = 0x7FFFFFFFll;

int32_t check_block(const char *fn, int32_t block_n, int32_t block_k) {
    if (block_n <= 0 || block_k <= 0)
        return fail(BI8_ERR_BLOCK, "%s: block size [%d, %d] must be two positive integers", fn,
                    block_n, block_k);
    if (block_n != 128 || block_k != 128)
        return fail(BI8_ERR_BLOCK, "%s: only the [128, 128] block is implemented, got [%d, %d]",
                    fn, block_n, block_k);
    return BI8_OK;
}

// The per-channel form of the method is the degenerate block (1, K): one
// scale per weight row and one per token.  Its int32 sums span all of K.
constexpr int64_t kMaxPerChannelK = 1 << 17;   // 127^2 * 2^17 < 2^31

bool per_channel(int32_t block_n, int32_t block_k, int64_t K) { return block_n == 1 && block_k == K; }

int32_t check_k(const char *fn, int64_t K) {
    if (K <= 0 || K > BI8_MAX_K)
        return fail(BI8_ERR_SHAPE, "%s: K = %lld out of range [1, %d]", fn, (long long)K, BI8_MAX_K);
    return BI8_OK;
}

// The steps whose kernels move rows in 16-byte pieces only (the grouped GEMM,
// the SiLU requantisation, the weight quantiser) need K % 16 == 0.
int32_t check_k16(const char *fn, int64_t K) {
    int32_t s = check_k(fn, K);
    if (s) return s;
    if (K % 16 != 0)
        return fail(BI8_ERR_ALIGN, "%s: K = %lld must be a multiple of 16", fn, (long long)K);
    return BI8_OK;
}

int32_t hip_status(const char *fn, hipError_t e) {
    if (e != hipSuccess) return fail(BI8_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return ok();
}

// Checks shared by the dense and grouped GEMM (allow_pc: the per-channel
// block (1, K) is accepted too).
int32_t check_gemm_common(const char *fn, const int8_t *xq, const float *xs, const int8_t *w,
                          const float *ws, const uint16_t *y, int64_t rows, int64_t N, int64_t K,
                          int32_t block_n, int32_t block_k, bool allow_pc = false, bool need_k16 = false) {
    if (rows < 0 || rows > kMaxRows)
        return fail(BI8_ERR_SHAPE, "%s: row count %lld out of range", fn, (long long)rows);
    if (N <= 0 || N > kMaxRows)
        return fail(BI8_ERR_SHAPE, "%s: N = %lld out of range", fn, (long long)N);
    int32_t s = need_k16 ? check_k16(fn, K) : check_k(fn, K);
    if (s) return s;
    if (allow_pc && per_channel(block_n, block_k, K)) {
        if (K > kMaxPerChannelK)
            return fail(BI8_ERR_SHAPE, "%s: per-channel blocks take K <= %lld, got %lld", fn,
                        (long long)kMaxPerChannelK, (long long)K);
    } else if ((s = check_block(fn, block_n, block_k))) {
        return s;
    }
    if (rows == 0) return BI8_OK;
    if (!xq || !xs || !w || !ws || !y) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(xq, 16) || !aligned(w, 16))
        return fail(BI8_ERR_ALIGN, "%s: xq and w must be 16-byte aligned", fn);
    if (!aligned(xs, 4) || !aligned(ws, 4))
        return fail(BI8_ERR_ALIGN, "%s: xs and ws must be 4-byte aligned", fn);
    if (!aligned(y, 2)) return fail(BI8_ERR_ALIGN, "%s: y must be 2-byte aligned", fn);
    return BI8_OK;
}

}  // namespace

namespace bi8 {

int32_t fail_status(int32_t status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int32_t call_status(const char *fn, hipError_t e) { return hip_status(fn, e); }

// Argument checks of the dynamic-scale linear (blockint8_linear and its
// allocation-free form), workspaces aside.
int32_t check_linear_args(const char *fn, const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                          const uint16_t *bias, const uint16_t *y, int64_t M, int64_t N, int64_t K,
                          int32_t block_n, int32_t block_k) {
    if (M < 0 || M > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: M = %lld out of range", fn, (long long)M);
    if (N <= 0 || N > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: N = %lld out of range", fn, (long long)N);
    int32_t s = check_k(fn, K);
    if (s) return s;
    if (ldx < K) return fail(BI8_ERR_SHAPE, "%s: ldx = %lld < K = %lld", fn, (long long)ldx, (long long)K);
    const bool pc = per_channel(block_n, block_k, K);
    if (pc && K > kMaxPerChannelK)
        return fail(BI8_ERR_SHAPE, "%s: per-channel blocks take K <= %lld, got %lld", fn,
                    (long long)kMaxPerChannelK, (long long)K);
    if (!pc && (s = check_block(fn, block_n, block_k))) return s;
    if (M == 0) return BI8_OK;
    if (!x || !w || !ws || !y) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(x, 2)) return fail(BI8_ERR_ALIGN, "%s: x must be 2-byte aligned", fn);
    if (!aligned(w, 16)) return fail(BI8_ERR_ALIGN, "%s: w must be 16-byte aligned", fn);
    if (!aligned(ws, 4)) return fail(BI8_ERR_ALIGN, "%s: ws must be 4-byte aligned", fn);
    if (!aligned(y, 2) || (bias && !aligned(bias, 2)))
        return fail(BI8_ERR_ALIGN, "%s: y and bias must be 2-byte aligned", fn);
    return BI8_OK;
}

// The two launches of the linear: quantise x into (xq, xs), then the GEMM.
hipError_t launch_linear(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws, const uint16_t *bias,
                         uint16_t *y, int64_t M, int64_t N, int64_t K, int32_t block_n, int32_t block_k,
                         int8_t *xq, float *xs, hipStream_t st) {
    hipError_t e;
    if (per_channel(block_n, block_k, K)) {
        e = launch_quant_act_per_token(x, M, K, ldx, xq, xs, st);
        if (e == hipSuccess) e = launch_gemm_per_channel(xq, xs, w, ws, bias, y, M, N, K, st);
    } else {
        e = launch_quant_act(x, M, K, ldx, xq, xs, st);
        if (e == hipSuccess) e = launch_gemm(GemmPath::kAuto, xq, xs, w, ws, bias, y, M, N, K, st);
    }
    return e;
}

}  // namespace bi8

extern "C" {

const char *blockint8_status_string(int32_t status) {
    switch (status) {
        case BI8_OK: return "BI8_OK";
        case BI8_ERR_NULL: return "BI8_ERR_NULL";
        case BI8_ERR_SHAPE: return "BI8_ERR_SHAPE";
        case BI8_ERR_BLOCK: return "BI8_ERR_BLOCK";
        case BI8_ERR_ALIGN: return "BI8_ERR_ALIGN";
        case BI8_ERR_HIP: return "BI8_ERR_HIP";
        default: return "BI8_ERR_UNKNOWN";
    }
}

const char *blockint8_last_error(void) { return g_last_error; }

int32_t blockint8_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int32_t block_k,
                            int8_t *xq, float *xs, void *stream) {
    static const char fn[] = "blockint8_quant_act";
    if (M < 0 || M > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: M = %lld out of range", fn, (long long)M);
    int32_t s = check_k(fn, K);
    if (s) return s;
    if (ldx < K) return fail(BI8_ERR_SHAPE, "%s: ldx = %lld < K = %lld", fn, (long long)ldx, (long long)K);
    const bool per_token = block_k == K && block_k != 128;   // the per-channel form: one group per row
    if (!per_token && (s = check_block(fn, 128, block_k))) return s;
    if (M == 0) return ok();
    if (!x || !xq || !xs) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(x, 2)) return fail(BI8_ERR_ALIGN, "%s: x must be 2-byte aligned", fn);
    if (!aligned(xq, 16)) return fail(BI8_ERR_ALIGN, "%s: xq must be 16-byte aligned", fn);
    if (!aligned(xs, 4)) return fail(BI8_ERR_ALIGN, "%s: xs must be 4-byte aligned", fn);
    if (per_token)
        return hip_status(fn, bi8::launch_quant_act_per_token(x, M, K, ldx, xq, xs,
                                                               static_cast<hipStream_t>(stream)));
    return hip_status(fn, bi8::launch_quant_act(x, M, K, ldx, xq, xs,
                                                 static_cast<hipStream_t>(stream)));
}

int32_t blockint8_gemm_select(int64_t M, int64_t N, int64_t K) {
    return static_cast<int32_t>(bi8::select_gemm_path(M, N, K));
}

int32_t blockint8_moe_gemm_select(int64_t R, int64_t N, int64_t K, int32_t E) {
    return static_cast<int32_t>(bi8::select_moe_gemm_path(R, N, K, E));
}

int32_t blockint8_gemm_variant(int32_t variant, const int8_t *xq, const float *xs,
                               const int8_t *w, const float *ws, const uint16_t *bias,
                               uint16_t *y, int64_t M, int64_t N, int64_t K, int32_t block_n,
                               int32_t block_k, void *stream) {
    static const char fn[] = "blockint8_gemm";
    if (variant < BI8_GEMM_AUTO || variant > BI8_GEMM_TILE_256X256)
        return fail(BI8_ERR_SHAPE, "%s: unknown kernel variant %d", fn, variant);
    int32_t s = check_gemm_common(fn, xq, xs, w, ws, y, M, N, K, block_n, block_k, true);
    if (s) return s;
    const bool pc = per_channel(block_n, block_k, K);
    if (pc && variant != BI8_GEMM_AUTO)
        return fail(BI8_ERR_SHAPE, "%s: the per-channel form has one kernel (variant must be AUTO)", fn);
    if (K % 16 != 0 && variant != BI8_GEMM_AUTO)
        return fail(BI8_ERR_ALIGN, "%s: K = %lld is not a multiple of 16; that form has one kernel "
                    "(variant must be AUTO)", fn, (long long)K);
    if (variant == BI8_GEMM_SKINNY && M > 64)
        return fail(BI8_ERR_SHAPE, "%s: the skinny kernel takes M <= 64, got %lld", fn, (long long)M);
    if (M == 0) return ok();
    if (bias && !aligned(bias, 2)) return fail(BI8_ERR_ALIGN, "%s: bias must be 2-byte aligned", fn);
    if (pc)
        return hip_status(fn, bi8::launch_gemm_per_channel(xq, xs, w, ws, bias, y, M, N, K,
                                                            static_cast<hipStream_t>(stream)));
    return hip_status(fn, bi8::launch_gemm(static_cast<bi8::GemmPath>(variant), xq, xs, w, ws, bias,
                                           y, M, N, K, static_cast<hipStream_t>(stream)));
}

int32_t blockint8_gemm(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                       const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                       int32_t block_n, int32_t block_k, void *stream) {
    return blockint8_gemm_variant(BI8_GEMM_AUTO, xq, xs, w, ws, bias, y, M, N, K, block_n, block_k,
                                  stream);
}

int64_t blockint8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t block_n, int32_t block_k) {
    if (M <= 0 || M > kMaxRows || N <= 0 || N > kMaxRows || K <= 0 || K > BI8_MAX_K) return 0;
    if (block_n != 128 || block_k != 128) return 0;   // the per-channel form never splits K
    return bi8::splitk_workspace_bytes(M, N, K);
}

int32_t blockint8_gemm_ws(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                          const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K, int32_t block_n,
                          int32_t block_k, void *workspace, int64_t workspace_bytes, void *stream) {
    static const char fn[] = "blockint8_gemm_ws";
    int32_t s = check_gemm_common(fn, xq, xs, w, ws, y, M, N, K, block_n, block_k, true);
    if (s) return s;
    if (workspace_bytes < 0)
        return fail(BI8_ERR_SHAPE, "%s: workspace_bytes = %lld < 0", fn, (long long)workspace_bytes);
    if (M == 0) return ok();
    if (bias && !aligned(bias, 2)) return fail(BI8_ERR_ALIGN, "%s: bias must be 2-byte aligned", fn);
    if (workspace && !aligned(workspace, 16)) return fail(BI8_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (per_channel(block_n, block_k, K))
        return hip_status(fn, bi8::launch_gemm_per_channel(xq, xs, w, ws, bias, y, M, N, K, st));
    return hip_status(fn, bi8::launch_gemm_ws(xq, xs, w, ws, bias, y, M, N, K, static_cast<float *>(workspace),
                                              workspace ? workspace_bytes : 0, st));
}

int32_t blockint8_linear(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                         const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                         int32_t block_n, int32_t block_k, int8_t *xq_workspace,
                         float *xs_workspace, void *stream) {
    static const char fn[] = "blockint8_linear";
    int32_t s = bi8::check_linear_args(fn, x, ldx, w, ws, bias, y, M, N, K, block_n, block_k);
    if (s) return s;
    if (M == 0) return ok();
    if (!xq_workspace || !xs_workspace) return fail(BI8_ERR_NULL, "%s: NULL workspace pointer", fn);
    if (!aligned(xq_workspace, 16) || !aligned(xs_workspace, 4))
        return fail(BI8_ERR_ALIGN, "%s: xq workspace must be 16-byte and xs workspace 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_linear(x, ldx, w, ws, bias, y, M, N, K, block_n, block_k, xq_workspace,
                                             xs_workspace, static_cast<hipStream_t>(stream)));
}

int32_t blockint8_moe_gemm_variant(int32_t variant, const int8_t *xq, const float *xs,
                                   const int32_t *expert_offsets, const int8_t *w,
                                   const float *ws, uint16_t *y, int64_t R, int64_t N, int64_t K,
                                   int32_t E, int32_t block_n, int32_t block_k, void *stream) {
    static const char fn[] = "blockint8_moe_gemm";
    if (variant != BI8_GEMM_AUTO && variant != BI8_GEMM_TILE_256X128 && variant != BI8_GEMM_TILE_256X256)
        return fail(BI8_ERR_SHAPE, "%s: kernel variant %d does not run the grouped GEMM", fn, variant);
    if (E <= 0 || E > 65536) return fail(BI8_ERR_SHAPE, "%s: E = %d out of range [1, 65536]", fn, E);
    int32_t s = check_gemm_common(fn, xq, xs, w, ws, y, R, N, K, block_n, block_k, false, true);
    if (s) return s;
    if (R == 0) return ok();
    if (!expert_offsets) return fail(BI8_ERR_NULL, "%s: NULL expert_offsets", fn);
    if (!aligned(expert_offsets, 4))
        return fail(BI8_ERR_ALIGN, "%s: expert_offsets must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_moe_gemm(static_cast<bi8::GemmPath>(variant), xq, xs,
                                               expert_offsets, w, ws, y, R, N, K, E,
                                               static_cast<hipStream_t>(stream)));
}

int64_t blockint8_moe_gemm_workspace_size(int64_t R, int64_t N, int64_t K, int32_t E, int32_t block_n,
                                          int32_t block_k) {
    if (R <= 0 || R > kMaxRows || N <= 0 || N > kMaxRows || K <= 0 || K % 16 != 0 || E <= 0 || E > 65536 ||
        block_n != 128 || block_k != 128)
        return 0;
    return bi8::moe_gemm_workspace_bytes(R, N, K, E);
}

int32_t blockint8_moe_gemm_ws(const int8_t *xq, const float *xs, const int32_t *expert_offsets, const int8_t *w,
                              const float *ws, uint16_t *y, int64_t R, int64_t N, int64_t K, int32_t E,
                              int32_t block_n, int32_t block_k, void *workspace, int64_t workspace_bytes,
                              void *stream) {
    static const char fn[] = "blockint8_moe_gemm_ws";
    if (E <= 0 || E > 65536) return fail(BI8_ERR_SHAPE, "%s: E = %d out of range [1, 65536]", fn, E);
    int32_t s = check_gemm_common(fn, xq, xs, w, ws, y, R, N, K, block_n, block_k, false, true);
    if (s) return s;
    if (workspace_bytes < 0) return fail(BI8_ERR_SHAPE, "%s: workspace_bytes < 0", fn);
    if (workspace && !aligned(workspace, 16))
        return fail(BI8_ERR_ALIGN, "%s: the workspace must be 16-byte aligned", fn);
    if (R == 0) return ok();
    if (!expert_offsets) return fail(BI8_ERR_NULL, "%s: NULL expert_offsets", fn);
    if (!aligned(expert_offsets, 4))
        return fail(BI8_ERR_ALIGN, "%s: expert_offsets must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_moe_gemm_ws(xq, xs, expert_offsets, w, ws, y, R, N, K, E,
                                                  static_cast<float *>(workspace), workspace_bytes,
                                                  static_cast<hipStream_t>(stream)));
}

int32_t blockint8_moe_gemm(const int8_t *xq, const float *xs, const int32_t *expert_offsets,
                           const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N,
                           int64_t K, int32_t E, int32_t block_n, int32_t block_k, void *stream) {
    return blockint8_moe_gemm_variant(BI8_GEMM_AUTO, xq, xs, expert_offsets, w, ws, y, R, N, K, E,
                                      block_n, block_k, stream);
}

int32_t blockint8_quant_weight(const uint16_t *w, int64_t N, int64_t K, int64_t ldw, int32_t block_n,
                               int32_t block_k, int8_t *wq, float *ws, void *stream) {
    static const char fn[] = "blockint8_quant_weight";
    if (N < 0 || N > 65535ll * 128) return fail(BI8_ERR_SHAPE, "%s: N = %lld out of range", fn, (long long)N);
    int32_t s = check_k16(fn, K);
    if (s) return s;
    if (ldw < K) return fail(BI8_ERR_SHAPE, "%s: ldw = %lld < K = %lld", fn, (long long)ldw, (long long)K);
    if ((s = check_block(fn, block_n, block_k))) return s;
    if (N == 0) return ok();
    if (!w || !wq || !ws) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (ldw % 8 != 0) return fail(BI8_ERR_ALIGN, "%s: ldw = %lld must be a multiple of 8", fn, (long long)ldw);
    if (!aligned(w, 16) || !aligned(wq, 16)) return fail(BI8_ERR_ALIGN, "%s: w and wq must be 16-byte aligned", fn);
    if (!aligned(ws, 4)) return fail(BI8_ERR_ALIGN, "%s: ws must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_quant_weight(w, N, K, ldw, wq, ws, static_cast<hipStream_t>(stream)));
}

// Section 3 of the page: a block-quantised weight may be cut between
// tensor-parallel ranks only where a cut cannot split a scale block.  Every
// shard edge along a split axis is walked and tested against the block edge
// of that axis: block_k columns on the input axis, block_n rows on the
// output axis.
int32_t blockint8_check_tp_partition(int64_t input_size, int64_t input_size_per_partition,
                                     const int64_t *output_partition_sizes, int32_t n_out,
                                     int32_t tp_size, int32_t block_n, int32_t block_k) {
    static const char fn[] = "blockint8_check_tp_partition";
    if (block_n <= 0 || block_k <= 0 || tp_size <= 0 || input_size <= 0 || input_size_per_partition <= 0 ||
        n_out < 0)
        return fail(BI8_ERR_SHAPE, "%s: sizes, tp_size and block dimensions must be positive", fn);
    if (n_out > 0 && !output_partition_sizes) return fail(BI8_ERR_NULL, "%s: NULL output_partition_sizes", fn);

    // Input axis: the row-parallel layout hands each of the tp_size ranks a
    // run of input_size_per_partition columns (the ranks' runs make up the
    // input, up to the rounding of the division); rank r's run starts at
    // column r * input_size_per_partition.  In any other layout the input
    // axis is not cut.
    const bool input_axis_cut = tp_size > 1 && input_size / input_size_per_partition == tp_size;
    for (int32_t r = 1; input_axis_cut && r < tp_size; ++r) {
        const int64_t first_col = (int64_t)r * input_size_per_partition;
        if (first_col % block_k != 0)
            return fail(BI8_ERR_BLOCK,
                        "%s: rank %d's input columns start at %lld, inside a scale block of %d columns "
                        "(input_size_per_partition = %lld)",
                        fn, r, (long long)first_col, block_k, (long long)input_size_per_partition);
    }

    // Output axis: the output partitions sit end to end along the weight's
    // rows (e.g. the fused gate and up projections); the row after each one
    // must start a scale block.
    int64_t next_row = 0;
    for (int32_t i = 0; i < n_out; ++i) {
        const int64_t rows = output_partition_sizes[i];
        if (rows <= 0)
            return fail(BI8_ERR_SHAPE, "%s: output partition %d has %lld rows", fn, i, (long long)rows);
        next_row += rows;
        if (next_row % block_n != 0)
            return fail(BI8_ERR_BLOCK,
                        "%s: output partition %d (%lld rows) ends inside a scale block of %d rows "
                        "(its last row is %lld)",
                        fn, i, (long long)rows, block_n, (long long)(next_row - 1));
    }
    return ok();
}

int32_t blockint8_moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                            int32_t *topk_ids, float *topk_weights, int32_t *sorted_token,
                            int32_t *expert_offsets, int32_t *row_of, void *stream) {
    static const char fn[] = "blockint8_moe_route";
    if (E < 1 || E > 1024) return fail(BI8_ERR_SHAPE, "%s: E = %d out of range [1, 1024]", fn, E);
    if (k < 1 || k > 8 || k > E) return fail(BI8_ERR_SHAPE, "%s: k = %d out of range [1, min(E, 8)]", fn, k);
    if (T < 0 || T * k > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: T = %lld out of range", fn, (long long)T);
    if (!expert_offsets) return fail(BI8_ERR_NULL, "%s: NULL expert_offsets", fn);
    if (T > 0 && (!logits || !topk_ids || !topk_weights || !sorted_token || !row_of))
        return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(expert_offsets, 4) ||
        (T > 0 && (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
                   !aligned(sorted_token, 4) || !aligned(row_of, 4))))
        return fail(BI8_ERR_ALIGN, "%s: pointers must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_moe_route(logits, T, E, k, renormalize, topk_ids, topk_weights,
                                                sorted_token, expert_offsets, row_of,
                                                static_cast<hipStream_t>(stream)));
}

int32_t blockint8_quant_act_gather(const uint16_t *x, int64_t T, int64_t ldx, const int32_t *rows,
                                   int64_t R, int64_t K, int32_t block_k, int8_t *xq, float *xs,
                                   void *stream) {
    static const char fn[] = "blockint8_quant_act_gather";
    if (R < 0 || R > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: R = %lld out of range", fn, (long long)R);
    if (T < 0) return fail(BI8_ERR_SHAPE, "%s: T = %lld < 0", fn, (long long)T);
    int32_t s = check_k(fn, K);
    if (s) return s;
    if (ldx < K) return fail(BI8_ERR_SHAPE, "%s: ldx = %lld < K = %lld", fn, (long long)ldx, (long long)K);
    if ((s = check_block(fn, 128, block_k))) return s;
    if (R == 0) return ok();
    if (!rows || !xq || !xs || (T > 0 && !x)) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (x && !aligned(x, 2)) return fail(BI8_ERR_ALIGN, "%s: x must be 2-byte aligned", fn);
    if (!aligned(xq, 16)) return fail(BI8_ERR_ALIGN, "%s: xq must be 16-byte aligned", fn);
    if (!aligned(xs, 4) || !aligned(rows, 4)) return fail(BI8_ERR_ALIGN, "%s: xs and rows must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_quant_act_gather(x, T, ldx, rows, R, K, xq, xs,
                                                        static_cast<hipStream_t>(stream)));
}

int32_t blockint8_moe_gemm_silu_quant(const int8_t *xq, const float *xs, const int32_t *expert_offsets,
                                      const int8_t *w13, const float *ws13, int8_t *aq, float *as, int64_t R,
                                      int64_t I, int64_t K, int32_t E, int32_t block_n, int32_t block_k,
                                      void *stream) {
    static const char fn[] = "blockint8_moe_gemm_silu_quant";
    if (E <= 0 || E > 65536) return fail(BI8_ERR_SHAPE, "%s: E = %d out of range [1, 65536]", fn, E);
    if (I <= 0 || I % 128 != 0 || I > kMaxRows / 2)
        return fail(BI8_ERR_SHAPE, "%s: I = %lld must be a positive multiple of 128", fn, (long long)I);
    // a placeholder y: the epilogue writes aq / as, no bf16 output
    const uint16_t *no_y = reinterpret_cast<const uint16_t *>(aq);
    int32_t s = check_gemm_common(fn, xq, xs, w13, ws13, no_y, R, 2 * I, K, block_n, block_k, false, true);
    if (s) return s;
    if (R == 0) return ok();
    if (!expert_offsets || !aq || !as) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(expert_offsets, 4))
        return fail(BI8_ERR_ALIGN, "%s: expert_offsets must be 4-byte aligned", fn);
    if (!aligned(aq, 16)) return fail(BI8_ERR_ALIGN, "%s: aq must be 16-byte aligned", fn);
    if (!aligned(as, 4)) return fail(BI8_ERR_ALIGN, "%s: as must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_moe_gemm_silu_quant(xq, xs, expert_offsets, w13, ws13, aq, as, R, I, K, E,
                                                          static_cast<hipStream_t>(stream)));
}

int32_t blockint8_silu_mul_quant(const uint16_t *h, int64_t R, int64_t I, int32_t block_k, int8_t *aq,
                                 float *as, uint16_t *a, void *stream) {
    static const char fn[] = "blockint8_silu_mul_quant";
    if (R < 0 || R > kMaxRows) return fail(BI8_ERR_SHAPE, "%s: R = %lld out of range", fn, (long long)R);
    int32_t s = check_k16(fn, I);
    if (s) return s;
    if ((s = check_block(fn, 128, block_k))) return s;
    if (R == 0) return ok();
    if (!h || !aq || !as) return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned(h, 16) || !aligned(aq, 16) || (a && !aligned(a, 16)))
        return fail(BI8_ERR_ALIGN, "%s: h, aq and a must be 16-byte aligned", fn);
    if (!aligned(as, 4)) return fail(BI8_ERR_ALIGN, "%s: as must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_silu_mul_quant(h, R, I, aq, as, a, static_cast<hipStream_t>(stream)));
}

int32_t blockint8_moe_combine(const uint16_t *y2, int64_t R, const int32_t *row_of,
                              const float *topk_weights, int64_t T, int32_t k, int64_t H,
                              uint16_t *out, void *stream) {
    static const char fn[] = "blockint8_moe_combine";
    if (T < 0 || R < 0 || R > kMaxRows || H <= 0 || H > kMaxRows || k < 1 || T * k > kMaxRows)
        return fail(BI8_ERR_SHAPE, "%s: bad shape T = %lld, R = %lld, k = %d, H = %lld", fn, (long long)T,
                    (long long)R, k, (long long)H);
    if (H % 8 != 0) return fail(BI8_ERR_ALIGN, "%s: H = %lld must be a multiple of 8", fn, (long long)H);
    if (T == 0) return ok();
    if (!row_of || !topk_weights || !out || (R > 0 && !y2))
        return fail(BI8_ERR_NULL, "%s: NULL tensor pointer", fn);
    if ((y2 && !aligned(y2, 16)) || !aligned(out, 16))
        return fail(BI8_ERR_ALIGN, "%s: y2 and out must be 16-byte aligned", fn);
    if (!aligned(row_of, 4) || !aligned(topk_weights, 4))
        return fail(BI8_ERR_ALIGN, "%s: row_of and weights must be 4-byte aligned", fn);
    return hip_status(fn, bi8::launch_moe_combine(y2, R, row_of, topk_weights, T, k, H, out,
                                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
