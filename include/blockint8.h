/*
 * blockint8.h -- C ABI of the block-wise INT8 W8A8 linear layer for AMD
 * Instinct MI355X (gfx950, CDNA4).
 *
 * The method (page "[SGLang] Block-wise INT8: 블록 단위 정수 양자화",
 * blog.secrett2633.cloud):
 *   - weights are int8 [N, K] (output dim first) with one fp32 scale per
 *     block_n x block_k block, scale tensor [ceil(N/block_n), ceil(K/block_k)]
 *     (structure diagram; section 2 and its worked example);
 *   - activations are quantised at run time, per token, with no static input
 *     scale (section 4; section 1 allows only the dynamic scheme); one fp32
 *     scale per (token, group of block_k consecutive K entries);
 *   - the GEMM multiplies int8 by int8, sums exactly inside each K block and
 *     rescales each block sum by activation scale x weight scale in fp32
 *     (design rationale item 3: fp32 scales, multiplied on dequantisation);
 *   - the MoE form keeps one int8 weight and one scale tensor per expert on a
 *     leading expert axis (sections 5 and 6).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     owned by the caller; tensors are row-major and dense unless a leading
 *     dimension is given.  bf16 values are passed as their uint16_t bits.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; nothing is synchronised.
 *   - The library allocates no device memory and keeps no state between
 *     calls apart from a thread-local error message.
 *   - Every argument is checked on the host before any HIP call; a failed
 *     check returns a status below and enqueues nothing.  BI8_ERR_HIP means a
 *     HIP call (the launch) failed; see blockint8_last_error().
 *   - This library implements the [128, 128] block, the block the pages
 *     describe as the usual one (design rationale item 1); any other positive
 *     block size returns BI8_ERR_BLOCK.
 *   - K is any size from 1 (section 2 sizes the scale tensor with a ceiling
 *     for any input size): the activation quantisation, the GEMM and the
 *     linear take any K and any row stride.  The kernels move int8 rows in
 *     16-byte pieces; with K % 16 != 0 the rows start at any byte, and one
 *     alignment-safe kernel serves every shape (slower than the tiled kernels
 *     of K % 16 == 0).  The grouped GEMM, the SiLU requantisation and the
 *     weight quantiser keep K % 16 == 0.  N and M are arbitrary.  Empty
 *     inputs (M == 0, R == 0) are a no-op.
 */
#ifndef BLOCKINT8_H_
#define BLOCKINT8_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bi8_status {
    BI8_OK = 0,
    BI8_ERR_NULL = 1,   /* a required pointer is NULL                          */
    BI8_ERR_SHAPE = 2,  /* a size is out of range (negative, zero, ldx < K, ...) */
    BI8_ERR_BLOCK = 3,  /* block size not positive, or not [128, 128]           */
    BI8_ERR_ALIGN = 4,  /* pointer / leading dimension / K alignment violated   */
    BI8_ERR_HIP = 5     /* a HIP runtime call failed                            */
} bi8_status;

/* Largest K accepted (elements); M, N and R are bounded by 2^31 - 1. */
#define BI8_MAX_K (1 << 23)

/* Static, never-NULL name of a status code. */
const char *blockint8_status_string(int32_t status);

/* Human-readable detail of the last failing call made on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char *blockint8_last_error(void);

/*
 * Dynamic activation quantisation (section 4: per-token scales computed at
 * run time; design rationale item 3: int8 values, fp32 scales).
 *
 *   x   bf16 [M, ldx], the first K columns of each row are quantised (any
 *       row stride ldx >= K, x 2-byte aligned)
 *   xq  int8 [M, K]                    (output)
 *   xs  fp32 [M, ceil(K / block_k)]    (output)
 *
 * For token m and group g (columns [g*block_k, min(K, (g+1)*block_k))):
 *   amax = max |x|,  s = amax / 127 (binary32, round to nearest),
 *   xq = 0 if s == 0 else clamp(round_half_even(x / s), -127, 127),
 *   xs[m, g] = s.
 * Bit-exact for finite inputs: s is a correctly rounded division, and each
 * code equals round_half_even of the correctly rounded quotient x / s (it is
 * formed as x * (1/s), with the division itself wherever the two could round
 * apart); subnormals are kept.  Non-finite inputs give unspecified codes.
 *
 * block_k is 128, or K: one group per token, the per-token scales of the
 * per-channel W8A8 form (the w8a8_int8 scheme of the SGLang quantization
 * page's platform matrix), xs then [M, 1].
 *
 * Errors: NULL x/xq/xs (M > 0) -> BI8_ERR_NULL; M < 0, K <= 0, K > BI8_MAX_K,
 * ldx < K -> BI8_ERR_SHAPE; block_k not 128 or K -> BI8_ERR_BLOCK; x not
 * 2-byte aligned, xq not 16-byte aligned, xs not 4-byte aligned ->
 * BI8_ERR_ALIGN.
 */
int32_t blockint8_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            int32_t block_k, int8_t *xq, float *xs, void *stream);

/*
 * Block-scaled int8 GEMM, y = x . W^T (structure diagram and section 2: int8
 * weight [N, K] with fp32 block scales; section 4: the linear's inputs are
 * the weight, its block scales, dynamic activation scales and an optional
 * bias).
 *
 *   xq    int8 [M, K]                         (from blockint8_quant_act)
 *   xs    fp32 [M, ceil(K / block_k)]
 *   w     int8 [N, K]
 *   ws    fp32 [ceil(N / block_n), ceil(K / block_k)]
 *   bias  bf16 [N] or NULL
 *   y     bf16 [M, N]                         (output)
 *
 *   y[m, n] = bf16_rne( sum_g  (sum_{k in g} xq[m,k] * w[n,k])
 *                              * (xs[m, g] * ws[n / block_n, g])  (+ bias[n]) )
 * Block sums are exact int32; the rescaled sum is accumulated in fp32 (the
 * order of the fp32 additions is unspecified).
 *
 * Blocks are [128, 128], or [1, K]: the per-channel form (one scale per
 * weight row, ws [N, 1], and per token, xs [M, 1]), the degenerate block of
 * the same formula; its int32 sums span all of K, so K <= 2^17 there.
 *
 * Errors: NULL xq/xs/w/ws/y (M > 0) -> BI8_ERR_NULL; M < 0, N <= 0, K <= 0,
 * K > BI8_MAX_K (2^17 per-channel) -> BI8_ERR_SHAPE; blocks other than
 * [128, 128] and [1, K] -> BI8_ERR_BLOCK;
 * xq / w not 16-byte aligned, xs / ws not 4-byte aligned, y / bias not
 * 2-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_gemm(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                       const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                       int32_t block_n, int32_t block_k, void *stream);

/*
 * blockint8_gemm with an optional caller workspace (the library allocates
 * nothing).  On problems whose grid of tiles is smaller than the chip
 * (fewer than one 128 x 64 tile per compute unit, e.g. a few hundred tokens),
 * a workspace lets the K dimension be split between workgroups: each split
 * sums its own run of K blocks (exact int32 block sums, rescaled in fp32) into
 * fp32 partial sums in the workspace, and a second launch adds the splits in
 * a fixed order, adds the bias and rounds to bf16.  Results are deterministic
 * and equal blockint8_gemm's up to the order of the fp32 additions (exact
 * where the sums are, e.g. integer or power-of-two cases).
 *
 *   workspace        device memory, 16-byte aligned, or NULL; contents need
 *                    no initialisation and are undefined on return
 *   workspace_bytes  its size; when it is below
 *                    blockint8_gemm_workspace_size(M, N, K, ...) (or NULL),
 *                    the call is exactly blockint8_gemm
 *
 * Calls that share one workspace must not overlap in time.
 * Errors: as blockint8_gemm; workspace_bytes < 0 -> BI8_ERR_SHAPE;
 * workspace not 16-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_gemm_ws(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                          const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                          int32_t block_n, int32_t block_k, void *workspace, int64_t workspace_bytes,
                          void *stream);

/* Workspace bytes blockint8_gemm_ws uses for this problem (0: it never splits
 * K there, e.g. large grids, K % 16 != 0, the per-channel block, bad sizes). */
int64_t blockint8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t block_n, int32_t block_k);

/*
 * Grouped (FusedMoE) block-scaled int8 GEMM (section 5: per-expert int8
 * weights with per-expert fp32 block scales on a leading expert axis;
 * section 6: the MoE runner applies the int8 W8A8 block arithmetic per
 * expert).  Rows are the dispatched tokens, sorted by expert.
 *
 *   xq              int8 [R, K]
 *   xs              fp32 [R, ceil(K / block_k)]
 *   expert_offsets  int32 [E + 1] on the DEVICE: rows [off[e], off[e+1]) use
 *                   expert e.  Precondition (not read by the host, so not
 *                   checked): off[0] = 0, off[E] = R, non-decreasing.
 *   w               int8 [E, N, K]
 *   ws              fp32 [E, ceil(N / block_n), ceil(K / block_k)]
 *   y               bf16 [R, N]               (output)
 *
 * Each segment is blockint8_gemm with that expert's w[e], ws[e] (no bias).
 * Empty segments are allowed.
 *
 * Errors: as blockint8_gemm; NULL expert_offsets -> BI8_ERR_NULL;
 * E <= 0 or E > 65536, R < 0 -> BI8_ERR_SHAPE; K % 16 != 0 (the grouped
 * kernels are the tiled ones) or expert_offsets not 4-byte aligned ->
 * BI8_ERR_ALIGN.
 */
int32_t blockint8_moe_gemm(const int8_t *xq, const float *xs, const int32_t *expert_offsets,
                           const int8_t *w, const float *ws, uint16_t *y,
                           int64_t R, int64_t N, int64_t K, int32_t E,
                           int32_t block_n, int32_t block_k, void *stream);

/*
 * blockint8_moe_gemm with a caller workspace (section 6: the per-expert int8
 * GEMMs of the fused-MoE runner).  When the tiles do not fill whole rounds of
 * the chip's CUs, the tiles of the last, partial round run split over K into
 * units that fill a round, and a second launch adds each such tile's fp32
 * partial sums in split order and rounds to bf16 (deterministic; the other
 * tiles are computed exactly as by blockint8_moe_gemm, and the split tiles
 * differ from it only by the fp32 summation order).  The library still
 * allocates nothing.
 *
 *   arguments as blockint8_moe_gemm, plus
 *   workspace        device memory, 16-byte aligned, or NULL
 *   workspace_bytes  its size; with less than
 *                    blockint8_moe_gemm_workspace_size(R, N, K, E, 128, 128)
 *                    (or NULL) the call is blockint8_moe_gemm
 *
 * Calls that overlap in time must not share a workspace.  Errors: as
 * blockint8_moe_gemm; workspace_bytes < 0 -> BI8_ERR_SHAPE; a workspace not
 * 16-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_moe_gemm_ws(const int8_t *xq, const float *xs, const int32_t *expert_offsets,
                              const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N, int64_t K,
                              int32_t E, int32_t block_n, int32_t block_k, void *workspace,
                              int64_t workspace_bytes, void *stream);

/*
 * Workspace bytes blockint8_moe_gemm_ws can use for a grouped problem: a
 * fixed 32 MiB (one round of 256 x 128 fp32 partial tiles) when the grouped
 * GEMM runs its 256 x 128 kernel, else 0 (and 0 for arguments the GEMM
 * rejects).  A host rule: it reads no device memory.
 */
int64_t blockint8_moe_gemm_workspace_size(int64_t R, int64_t N, int64_t K, int32_t E, int32_t block_n,
                                          int32_t block_k);

/*
 * Dynamic-scale block-wise INT8 linear in one call: the activations are
 * quantised at run time (blockint8_quant_act) and fed to the block-scaled
 * GEMM (blockint8_gemm).  Section 4 of the page: the linear takes the input,
 * the int8 weight, its block scales and an optional bias, and with no input
 * scale it computes the per-token activation scales itself.
 *
 *   x             bf16 [M, ldx]; row stride ldx >= K elements, 2-byte aligned
 *   w, ws, bias, y, block_n, block_k: as blockint8_gemm
 *   xq_workspace  int8 [M, K]           caller-owned; hold the quantised
 *   xs_workspace  fp32 [M, ceil(K/128)] activations on return
 *
 * Two launches on the stream (quantisation, then the GEMM); y equals
 * blockint8_quant_act followed by blockint8_gemm exactly.
 *
 * Errors: as blockint8_quant_act and blockint8_gemm; NULL workspace ->
 * BI8_ERR_NULL; workspace misaligned (xq 16 B, xs 4 B) -> BI8_ERR_ALIGN.
 */
int32_t blockint8_linear(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                         const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                         int32_t block_n, int32_t block_k, int8_t *xq_workspace,
                         float *xs_workspace, void *stream);

/*
 * blockint8_linear without workspace arguments, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The library
 * allocates nothing either: the quantised activations and their scales are
 * staged in a fixed array of BI8_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on every GPU it runs on until the process ends.
 *
 *   x, ldx, w, ws, bias, y, M, N, K, block_n, block_k: as blockint8_linear
 *
 * Same launches and results as blockint8_linear (y bit-identical).  The
 * codes [M, K] and scales [M, ceil(K/128)] (per-channel: [M, 1]) must fit:
 * round_up(M * K, 256) + 4 * M * (number of K groups) <= 20 MiB, e.g. M * K
 * up to 16 MiB at K >= 256.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race and give
 * undefined results; calls on one stream are ordered and safe.  The first
 * call on a device looks the array's address up on that device (the calling
 * thread's current device, which must be the device of the pointers).
 *
 * Errors: as blockint8_linear; a problem larger than the array ->
 * BI8_ERR_SHAPE.
 */
#define BI8_NOALLOC_SCRATCH_BYTES (20ll << 20)

int32_t blockint8_linear_noalloc(const uint16_t *x, int64_t ldx, const int8_t *w, const float *ws,
                                 const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                 int32_t block_n, int32_t block_k, void *stream);

/*
 * Offline block quantisation of a bf16 weight into the int8 + fp32 block
 * scale form that blockint8_gemm consumes (section 1 of the page: only
 * int8-serialised weights are loaded; section 2: one fp32 scale per
 * (block_n x block_k) block, scale tensor [ceil(N/bn), ceil(K/bk)]).  Per
 * block: s = amax / 127, q = clamp(rne(w / s), -127, 127), 0 when s == 0 --
 * the same encoding as the activations, per 2-D block.
 *
 *   w   bf16 [N, ldw]  (ldw >= K, ldw % 8 == 0, 16-byte aligned)
 *   wq  int8 [N, K]    (16-byte aligned)   ws fp32 [ceil(N/128), ceil(K/128)]
 *
 * Limits: N <= 65535 * 128.  Errors: NULL pointer (N > 0) -> BI8_ERR_NULL;
 * N < 0, K <= 0, ldw < K, N too large -> BI8_ERR_SHAPE; block != [128, 128]
 * -> BI8_ERR_BLOCK; K % 16, ldw % 8 or alignment -> BI8_ERR_ALIGN.
 */
int32_t blockint8_quant_weight(const uint16_t *w, int64_t N, int64_t K, int64_t ldw, int32_t block_n,
                               int32_t block_k, int8_t *wq, float *ws, void *stream);

/*
 * Tensor-parallel partition check (section 3 of the page): with block
 * quantisation, a cut between ranks must not split a scale block.
 *   input axis:  when tp_size > 1 ranks each take input_size_per_partition
 *                columns (input_size / input_size_per_partition == tp_size,
 *                integer division), the first column of every rank after the
 *                first must be a multiple of block_k;
 *   output axis: the output partitions lie end to end along the rows, and
 *                each must end on a multiple of block_n rows.
 * Host only (no device pointer, no launch).  Returns BI8_OK, or
 * BI8_ERR_BLOCK with the offending shard edge in blockint8_last_error();
 * BI8_ERR_NULL / BI8_ERR_SHAPE for a NULL array with n_out > 0 or a
 * non-positive size.
 */
int32_t blockint8_check_tp_partition(int64_t input_size, int64_t input_size_per_partition,
                                     const int64_t *output_partition_sizes, int32_t n_out,
                                     int32_t tp_size, int32_t block_n, int32_t block_k);

/* ---------------------------------------------------------------------
 * The MoE steps on either side of the grouped GEMM (section 6 of the page:
 * the fused-MoE runner routes the tokens, runs the per-expert int8 GEMMs and
 * combines the expert outputs).  With them the whole FusedMoE layer runs on
 * the GPU:
 *
 *   blockint8_moe_route          logits -> top-k ids and weights, dispatch
 *                                order, expert_offsets, row_of
 *   blockint8_quant_act_gather   x[sorted_token] -> int8 rows + scales
 *   blockint8_moe_gemm           w13 (gate | up) per expert
 *   blockint8_silu_mul_quant     silu(gate) * up -> int8 rows + scales
 *   blockint8_moe_gemm           w2 per expert
 *   blockint8_moe_combine        weighted sum of each token's k rows
 *
 * blockint8_moe_gemm_silu_quant does the w13 GEMM and the activation step in
 * one launch (I % 128 == 0).
 * ------------------------------------------------------------------- */

/*
 * Router and dispatch order, two launches on the stream.
 *
 *   logits        fp32 [T, E] (device)
 *   topk_ids      int32 [T, k]  out: the k experts with the largest softmax
 *                 probability, in that order; ties go to the lower expert
 *   topk_weights  fp32 [T, k]   out: their probabilities (divided by their
 *                 sum when renormalize != 0)
 *   sorted_token  int32 [T*k]   out: token of each dispatched row; rows are
 *                 sorted stably by (expert, token)
 *   expert_offsets int32 [E+1]  out: rows [off[e], off[e+1]) use expert e
 *   row_of        int32 [T, k]  out: the row that (token, slot) went to
 *
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 8), T * k < 2^31.  T == 0 writes
 * expert_offsets (all zero).  Errors: NULL pointer -> BI8_ERR_NULL; a limit
 * broken -> BI8_ERR_SHAPE; a pointer not 4-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renormalize,
                            int32_t *topk_ids, float *topk_weights, int32_t *sorted_token,
                            int32_t *expert_offsets, int32_t *row_of, void *stream);

/*
 * blockint8_quant_act on gathered rows: output row r quantises row rows[r]
 * of x (the dispatch of the tokens to their expert rows; quantising per
 * token and gathering give the same codes, so this is exact).
 *
 *   x     bf16 [T, ldx]   rows int32 [R] on the device, values in [0, T)
 *                          (an index outside reads as an all-zero row)
 *   xq    int8 [R, K]      xs fp32 [R, ceil(K/128)]
 *
 * Errors: as blockint8_quant_act; NULL rows -> BI8_ERR_NULL; T < 0 ->
 * BI8_ERR_SHAPE.
 */
int32_t blockint8_quant_act_gather(const uint16_t *x, int64_t T, int64_t ldx, const int32_t *rows,
                                   int64_t R, int64_t K, int32_t block_k, int8_t *xq, float *xs,
                                   void *stream);

/*
 * Gate/up activation fused with the quantisation of its result, for the w2
 * GEMM.  h (the w13 output) holds gate in columns [0, I) and up in [I, 2I):
 *
 *   a[r, i] = bf16( silu(gate) * up ),  silu(z) = z / (1 + exp(-z))  (fp32;
 *             exp and the quotient through the hardware exp2 and
 *             reciprocal, so a may differ from a correctly rounded
 *             evaluation by one bf16 ulp in rare cases; the bf16 rounding is
 *             to nearest even, a NaN keeps an unspecified NaN pattern)
 *   aq, as  = blockint8_quant_act(a)   (bit for bit, on this a)
 *
 *   h   bf16 [R, 2I] (16-byte aligned)   aq int8 [R, I]   as fp32 [R, ceil(I/128)]
 *   a   bf16 [R, I]  optional copy of the activation (NULL: not written)
 *
 * Errors: NULL h/aq/as (R > 0) -> BI8_ERR_NULL; R < 0, I <= 0 -> BI8_ERR_SHAPE;
 * block_k != 128 -> BI8_ERR_BLOCK; I % 16, h/aq/a not 16-byte aligned, as not
 * 4-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_silu_mul_quant(const uint16_t *h, int64_t R, int64_t I, int32_t block_k, int8_t *aq,
                                 float *as, uint16_t *a, void *stream);

/*
 * The w13 grouped GEMM with the gate/up activation and its quantisation as
 * the GEMM's epilogue (section 5: per-expert w13 holds the gate and the up
 * projection; section 6: the runner applies the int8 block arithmetic per
 * expert and the activation between the two projections).  One launch
 * computes what blockint8_moe_gemm(xq, xs, expert_offsets, w13, ws13, h,
 * R, 2I, K, E) followed by blockint8_silu_mul_quant(h, R, I) computes, bit
 * for bit, without writing h:
 *
 *   xq, xs, expert_offsets  as blockint8_moe_gemm (K % 16 == 0)
 *   w13   int8 [E, 2I, K]: rows [0, I) gate, rows [I, 2I) up
 *   ws13  fp32 [E, 2I / 128, ceil(K / 128)]
 *   aq    int8 [R, I]   (output, 16-byte aligned)
 *   as    fp32 [R, I / 128]   (output)
 *
 * Errors: as blockint8_moe_gemm; NULL aq/as (R > 0) -> BI8_ERR_NULL;
 * I not a positive multiple of 128 -> BI8_ERR_SHAPE; aq not 16-byte or as
 * not 4-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_moe_gemm_silu_quant(const int8_t *xq, const float *xs, const int32_t *expert_offsets,
                                      const int8_t *w13, const float *ws13, int8_t *aq, float *as, int64_t R,
                                      int64_t I, int64_t K, int32_t E, int32_t block_n, int32_t block_k,
                                      void *stream);

/*
 * Weighted combine: out[t, :] = bf16( sum_s w[t, s] * y2[row_of[t, s], :] ),
 * summed in fp32 in slot order.
 *
 *   y2  bf16 [R, H]   row_of int32 [T, k]   topk_weights fp32 [T, k]
 *   out bf16 [T, H]   (row_of entries outside [0, R) contribute nothing)
 *
 * Errors: NULL pointer (T > 0) -> BI8_ERR_NULL; T < 0, R < 0, H <= 0, k < 1
 * -> BI8_ERR_SHAPE; H % 8, y2/out not 16-byte aligned, row_of / weights not
 * 4-byte aligned -> BI8_ERR_ALIGN.
 */
int32_t blockint8_moe_combine(const uint16_t *y2, int64_t R, const int32_t *row_of,
                              const float *topk_weights, int64_t T, int32_t k, int64_t H,
                              uint16_t *out, void *stream);

/*
 * Kernel variants.  blockint8_gemm and blockint8_moe_gemm choose a kernel by
 * shape; the *_variant entry points run a named one instead, with the same
 * arguments, results and errors, so that every kernel can be checked and
 * timed on any shape it accepts.  With K % 16 != 0 a single kernel runs
 * every shape and only BI8_GEMM_AUTO is accepted (BI8_ERR_ALIGN otherwise).  A variant that cannot run the shape
 * (BI8_GEMM_SKINNY with more than 64 rows, BI8_GEMM_SKINNY or
 * BI8_GEMM_TILE_128X64 for the grouped GEMM) returns BI8_ERR_SHAPE; an
 * unknown variant id returns BI8_ERR_SHAPE.  The per-channel form ([1, K]
 * blocks) has a single kernel: only BI8_GEMM_AUTO runs it.
 *
 *   BI8_GEMM_AUTO          the shape-based choice
 *   BI8_GEMM_SKINNY        M <= 64: weight rows streamed into registers
 *   BI8_GEMM_TILE_128X64   128 weight rows x 64 activation rows per workgroup
 *   BI8_GEMM_TILE_256X128  256 x 128
 *   BI8_GEMM_TILE_256X256  256 x 256
 */
enum {
    BI8_GEMM_AUTO = 0,
    BI8_GEMM_SKINNY = 1,
    BI8_GEMM_TILE_128X64 = 2,
    BI8_GEMM_TILE_256X128 = 3,
    BI8_GEMM_TILE_256X256 = 4
};

/* The variant blockint8_gemm runs for an M x N x K problem (M, N, K > 0). */
int32_t blockint8_gemm_select(int64_t M, int64_t N, int64_t K);

/* The variant blockint8_moe_gemm runs for R rows over E experts. */
int32_t blockint8_moe_gemm_select(int64_t R, int64_t N, int64_t K, int32_t E);

int32_t blockint8_gemm_variant(int32_t variant, const int8_t *xq, const float *xs,
                               const int8_t *w, const float *ws, const uint16_t *bias,
                               uint16_t *y, int64_t M, int64_t N, int64_t K,
                               int32_t block_n, int32_t block_k, void *stream);

int32_t blockint8_moe_gemm_variant(int32_t variant, const int8_t *xq, const float *xs,
                                   const int32_t *expert_offsets, const int8_t *w,
                                   const float *ws, uint16_t *y, int64_t R, int64_t N,
                                   int64_t K, int32_t E, int32_t block_n, int32_t block_k,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKINT8_H_ */
