/*
 * oracle.c -- the CPU oracle for the block-wise INT8 W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Plain scalar C, written from the
 * pages' description of the method and nothing else.  It shares no code,
 * header, table or helper with the HIP library, and only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it.
 *
 * Pages cited (by title and section):
 *   [BW8] "[SGLang] Block-wise INT8: 블록 단위 정수 양자화"
 *         (blog.secrett2633.cloud, opensource/sglang/blockwise-int8)
 *   [SQ]  "양자화 (Quantization)" -- the SGLang quantization page of the
 *         data-sketchers wiki (platform matrix and W8A8 notes)
 *
 * Precision.  Quantisation decides integers, so it runs in IEEE binary32 as
 * the stored fp32 scales dictate ([BW8], design rationale item 3: scales are
 * fp32).  The GEMM's block sums are exact integers; their rescaled sum is
 * taken in binary64 and rounded once to bf16, so the oracle gives the exact
 * value (to ~1e-15) that the fp32 kernels approximate.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FTZ/DAZ, default round-to-nearest-even mode).
 *
 * Return codes: 0 = ok, -1 = bad argument, -2 = non-finite input.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 <-> binary32/binary64                                           */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper half of a binary32 with the same bits, so the
 * widening is exact. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary64 value to the nearest bf16 (8 significant bits, exponent
 * range of binary32), ties to even, in ONE rounding step.  Written from the
 * IEEE-754 definition: find the quantum (weight of the last kept bit) of the
 * binade that holds |v|, scale by it, round to an integer with the default
 * ties-to-even mode, scale back. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int q = (e - 1) - 7;          /* quantum of an 8-bit significand */
    if (q < -133) q = -133;       /* bf16 subnormal quantum is 2^-133 */
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80u); /* overflow -> inf */
    float f = (float)r;           /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* Exposed for the pin tests. */
float oracle_bf16_to_f32(uint16_t b) { return bf16_bits_to_f32(b); }

/* ------------------------------------------------------------------ */
/* Scale-tensor shape                                                   */
/* ------------------------------------------------------------------ */

/* [BW8] §2 (weight and block-scale creation): the fp32 scale tensor of an
 * int8 weight [N, K] has one entry per (block_n x block_k) block, rounding
 * partial blocks up: [ceil(N/block_n), ceil(K/block_k)]. */
int oracle_scale_shape(int64_t N, int64_t K, int64_t block_n, int64_t block_k,
                       int64_t *rows, int64_t *cols)
{
    if (N < 0 || K < 0 || block_n <= 0 || block_k <= 0 || !rows || !cols) return -1;
    *rows = (N + block_n - 1) / block_n;
    *cols = (K + block_k - 1) / block_k;
    return 0;
}

/* ------------------------------------------------------------------ */
/* O1: dynamic activation quantisation                                  */
/* ------------------------------------------------------------------ */

/* [BW8] §4 (inference apply): with no static input scale the activation
 * scale is computed at run time, per token; [BW8] structure diagram and §1:
 * only the dynamic scheme exists; design rationale item 3: int8 range with
 * fp32 scales.  Reading taken: one scale per (token m, group g of block_k
 * consecutive K entries), the last group holding the K % block_k remainder.
 *
 *   amax   = max |x[m,k]| over the group                (exact)
 *   s      = amax / 127                                 (binary32, RN)
 *   q[m,k] = 0 if s == 0, else clamp(rne(x[m,k] / s), -127, 127)
 *
 * x is bf16 bits [M, ldx] (row stride ldx >= K); xq is int8 [M, K];
 * xs is fp32 [M, ceil(K/block_k)]. */
int oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                     int64_t block_k, int8_t *xq, float *xs)
{
    if (M < 0 || K < 0 || ldx < K || block_k <= 0) return -1;
    if ((M > 0 && K > 0) && (!x || !xq || !xs)) return -1;
    const int64_t KB = (K + block_k - 1) / block_k;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = x + m * ldx;
        for (int64_t g = 0; g < KB; ++g) {
            const int64_t k0 = g * block_k;
            const int64_t k1 = (k0 + block_k < K) ? k0 + block_k : K;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float v = bf16_bits_to_f32(row[k]);
                if (!isfinite(v)) return -2;
                float a = fabsf(v);
                if (a > amax) amax = a;
            }
            const float s = amax / 127.0f;
            xs[m * KB + g] = s;
            for (int64_t k = k0; k < k1; ++k) {
                float q = 0.0f;
                if (s != 0.0f) {
                    q = rintf(bf16_bits_to_f32(row[k]) / s);
                    if (q > 127.0f) q = 127.0f;
                    if (q < -127.0f) q = -127.0f;
                }
                xq[m * K + k] = (int8_t)q;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O2: block-scaled int8 GEMM                                           */
/* ------------------------------------------------------------------ */

/* [BW8] structure diagram and §2: weight int8 [N, K] (output dim 0, input
 * dim 1), scale fp32 [ceil(N/block_n), ceil(K/block_k)]; §4: the linear
 * takes the int8 weight, its block scales, the dynamic activation scales and
 * an optional bias; design rationale item 3: dequantisation multiplies by
 * the fp32 scales.  Reading taken (y = x . W^T):
 *
 *   y[m,n] = sum_g ( sum_{k in g} xq[m,k] * w[n,k] ) * xs[m,g] * ws[n/bn, g]
 *            (+ bias[n]),  rounded once to bf16
 *
 * The inner sums are exact integers; the outer sum runs in binary64 over
 * ascending g.  The result is written as binary64 (y64, may be NULL) and/or
 * bf16 bits (y16, may be NULL). */
static int gemm_core(const int8_t *xq, const float *xs, const int8_t *w,
                     const float *ws, const uint16_t *bias, double *y64,
                     uint16_t *y16, int64_t M, int64_t N, int64_t K,
                     int64_t block_n, int64_t block_k)
{
    if (M < 0 || N < 0 || K < 0 || block_n <= 0 || block_k <= 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!xq || !xs || !w || !ws || (!y64 && !y16)) return -1;
    const int64_t KB = (K + block_k - 1) / block_k;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const int64_t nb = n / block_n;
            double acc_y = 0.0;
            for (int64_t g = 0; g < KB; ++g) {
                const int64_t k0 = g * block_k;
                const int64_t k1 = (k0 + block_k < K) ? k0 + block_k : K;
                int64_t acc = 0;
                for (int64_t k = k0; k < k1; ++k)
                    acc += (int64_t)xq[m * K + k] * (int64_t)w[n * K + k];
                const double t = (double)xs[m * KB + g] * (double)ws[nb * KB + g];
                acc_y += (double)acc * t;
            }
            if (bias) acc_y += (double)bf16_bits_to_f32(bias[n]);
            if (y64) y64[m * N + n] = acc_y;
            if (y16) y16[m * N + n] = oracle_f64_to_bf16(acc_y);
        }
    }
    return 0;
}

int oracle_gemm(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                int64_t block_n, int64_t block_k)
{
    if (!y && M > 0 && N > 0) return -1;
    return gemm_core(xq, xs, w, ws, bias, NULL, y, M, N, K, block_n, block_k);
}

int oracle_gemm_f64(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                    const uint16_t *bias, double *y, int64_t M, int64_t N, int64_t K,
                    int64_t block_n, int64_t block_k)
{
    if (!y && M > 0 && N > 0) return -1;
    return gemm_core(xq, xs, w, ws, bias, y, NULL, M, N, K, block_n, block_k);
}

/* ------------------------------------------------------------------ */
/* O2 per expert: the grouped (FusedMoE) form                           */
/* ------------------------------------------------------------------ */

/* [BW8] §5 (MoE weights): every expert e owns an int8 weight and its own
 * fp32 block scales, stacked on a leading expert axis: w [E, N, K],
 * ws [E, ceil(N/bn), ceil(K/bk)]; §6: the MoE runner applies the same
 * int8 W8A8 block arithmetic per expert.  Rows arrive sorted by expert:
 * rows [off[e], off[e+1]) use expert e.  Each segment is O2 with that
 * expert's weight and scales.  off is a host array of E+1 entries with
 * off[0] = 0, off[E] = R, non-decreasing. */
int oracle_moe_gemm(const int8_t *xq, const float *xs, const int32_t *off,
                    const int8_t *w, const float *ws, uint16_t *y,
                    int64_t R, int64_t N, int64_t K, int64_t E,
                    int64_t block_n, int64_t block_k)
{
    if (R < 0 || N < 0 || K < 0 || E <= 0 || block_n <= 0 || block_k <= 0 || !off) return -1;
    if (off[0] != 0 || off[E] != R) return -1;
    for (int64_t e = 0; e < E; ++e)
        if (off[e + 1] < off[e]) return -1;
    const int64_t NB = (N + block_n - 1) / block_n;
    const int64_t KB = (K + block_k - 1) / block_k;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t r0 = off[e], rows = off[e + 1] - off[e];
        if (rows == 0) continue;
        int rc = oracle_gemm(xq + r0 * K, xs + r0 * KB, w + e * N * K, ws + e * NB * KB,
                             NULL, y + r0 * N, rows, N, K, block_n, block_k);
        if (rc) return rc;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3: the MoE steps on either side of the grouped GEMM                 */
/* ------------------------------------------------------------------ */

/* Router.  [BW8] §6 hands dispatch and combine to the fused-MoE runner;
 * the workload routes each token to the top k of the softmax of its router
 * logits.  Per token t, in binary64:
 *   p[e] = exp(l[e] - max_e l) / sum_e exp(l[e] - max_e l)  (sum ascending e)
 *   the k largest p, picked one at a time (ties to the lower expert index),
 *   weight = the chosen p, divided by the sum of the k chosen when renorm.
 * logits fp32 [T, E]; ids int32 [T, k] in pick order; weights binary64 [T, k]. */
int oracle_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t k, int renorm,
                        int32_t *ids, double *weights)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E || E > 4096) return -1;
    if (T > 0 && (!logits || !ids || !weights)) return -1;
    double p[4096];
    unsigned char taken[4096];
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        double mx = -INFINITY;
        for (int64_t e = 0; e < E; ++e) {
            if (!isfinite(l[e])) return -2;
            if ((double)l[e] > mx) mx = (double)l[e];
        }
        double sum = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - mx);
            sum += p[e];
        }
        for (int64_t e = 0; e < E; ++e) {
            p[e] /= sum;
            taken[e] = 0;
        }
        double chosen = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
            weights[t * k + j] = p[best];
            chosen += p[best];
        }
        if (renorm)
            for (int64_t j = 0; j < k; ++j) weights[t * k + j] /= chosen;
    }
    return 0;
}

/* Dispatch order: the T*k rows (t, slot) sorted stably by (expert, t, slot),
 * so that each expert's rows form one segment [offsets[e], offsets[e+1]).
 * sorted_token int32 [T*k]: the token of each row; offsets int32 [E+1];
 * row_of int32 [T*k]: the row that (t, slot) went to. */
int oracle_moe_align(const int32_t *ids, int64_t T, int64_t k, int64_t E,
                     int32_t *sorted_token, int32_t *offsets, int32_t *row_of)
{
    if (T < 0 || k <= 0 || E <= 0 || !offsets) return -1;
    if (T > 0 && (!ids || !sorted_token || !row_of)) return -1;
    for (int64_t i = 0; i < T * k; ++i)
        if (ids[i] < 0 || ids[i] >= E) return -1;
    int64_t r = 0;
    for (int64_t e = 0; e < E; ++e) {
        offsets[e] = (int32_t)r;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t s = 0; s < k; ++s)
                if (ids[t * k + s] == e) {
                    sorted_token[r] = (int32_t)t;
                    row_of[t * k + s] = (int32_t)r;
                    ++r;
                }
    }
    offsets[E] = (int32_t)r;
    return 0;
}

/* Gate/up activation.  [BW8] §5: the MoE w13 weight is the gate and up
 * projections fused, [2I, H], with 2 * ceil(I/bn) scale rows, so its output
 * h [R, 2I] holds gate in columns [0, I) and up in [I, 2I) (gate first, the
 * plainest reading).  The activation is SiLU gating, in binary64:
 *   a[r, i] = bf16_rne( silu(gate) * up ),  silu(z) = z / (1 + exp(-z)). */
int oracle_silu_mul(const uint16_t *h, int64_t R, int64_t I, uint16_t *a)
{
    if (R < 0 || I < 0) return -1;
    if (R > 0 && I > 0 && (!h || !a)) return -1;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t i = 0; i < I; ++i) {
            const double g = (double)bf16_bits_to_f32(h[r * 2 * I + i]);
            const double u = (double)bf16_bits_to_f32(h[r * 2 * I + I + i]);
            if (!isfinite(g) || !isfinite(u)) return -2;
            const double silu = g / (1.0 + exp(-g));
            a[r * I + i] = oracle_f64_to_bf16(silu * u);
        }
    return 0;
}

/* Combine: each token's output is the routing-weighted sum of its k expert
 * rows, in binary64 with the slots in ascending order, rounded once:
 *   out[t, :] = bf16_rne( sum_s w[t, s] * y2[row_of[t, s], :] ).
 * y2 bf16 [R, H]; row_of int32 [T, k] in [0, R); w fp32 [T, k] (the weights
 * the router produced). */
int oracle_combine(const uint16_t *y2, int64_t R, const int32_t *row_of, const float *w,
                   int64_t T, int64_t k, int64_t H, uint16_t *out)
{
    if (T < 0 || k <= 0 || H < 0 || R < 0) return -1;
    if (T > 0 && H > 0 && (!y2 || !row_of || !w || !out)) return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int64_t s = 0; s < k; ++s) {
                const int64_t r = row_of[t * k + s];
                if (r < 0 || r >= R) return -1;
                acc += (double)w[t * k + s] * (double)bf16_bits_to_f32(y2[r * H + c]);
            }
            out[t * H + c] = oracle_f64_to_bf16(acc);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Offline weight quantisation                                          */
/* ------------------------------------------------------------------ */

/* [BW8] §1: the method loads only int8-serialised weights; §2: one fp32
 * scale per (block_n x block_k) block of the [N, K] weight, scale tensor
 * [ceil(N/bn), ceil(K/bk)]; design rationale item 3: the scale multiplies
 * on dequantisation.  Producing such a checkpoint from a bf16 weight uses the
 * same symmetric encoding as the activations, per 2-D block:
 *   s = amax over the block / 127 (binary32),
 *   q = 0 if s == 0, else clamp(rne(w / s), -127, 127).
 * The blocks at the N and K ends are ragged.  w is bf16 bits [N, ldw]. */
int oracle_quant_weight(const uint16_t *w, int64_t N, int64_t K, int64_t ldw, int64_t block_n,
                        int64_t block_k, int8_t *wq, float *ws)
{
    if (N < 0 || K < 0 || ldw < K || block_n <= 0 || block_k <= 0) return -1;
    if (N > 0 && K > 0 && (!w || !wq || !ws)) return -1;
    const int64_t NB = (N + block_n - 1) / block_n, KB = (K + block_k - 1) / block_k;
    for (int64_t bn = 0; bn < NB; ++bn)
        for (int64_t bk = 0; bk < KB; ++bk) {
            const int64_t n0 = bn * block_n, n1 = (n0 + block_n < N) ? n0 + block_n : N;
            const int64_t k0 = bk * block_k, k1 = (k0 + block_k < K) ? k0 + block_k : K;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k) {
                    const float v = bf16_bits_to_f32(w[n * ldw + k]);
                    if (!isfinite(v)) return -2;
                    if (fabsf(v) > amax) amax = fabsf(v);
                }
            const float s = amax / 127.0f;
            ws[bn * KB + bk] = s;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k) {
                    float q = 0.0f;
                    if (s != 0.0f) {
                        q = rintf(bf16_bits_to_f32(w[n * ldw + k]) / s);
                        if (q > 127.0f) q = 127.0f;
                        if (q < -127.0f) q = -127.0f;
                    }
                    wq[n * K + k] = (int8_t)q;
                }
        }
    return 0;
}
