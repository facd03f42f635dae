// The MoE steps on either side of the grouped GEMM (gfx950).
//
// Page "[SGLang] Block-wise INT8" (blog.secrett2633.cloud): section 5 (the
// MoE w13 weight fuses the gate and up projections, [2I, H], so its output
// carries gate and up side by side) and section 6 (the fused-MoE runner
// dispatches the tokens to their experts, runs the per-expert int8 GEMMs and
// combines the results).  The workload routes each token to the top k of the
// softmax of its router logits.  Kernels:
//
//  * moe_topk_kernel     one thread per token: softmax in fp32 and the k
//                        largest, picked on the logits (the softmax is
//                        monotone, so the choice is exact; ties to the lower
//                        expert), weights exp(l - max) / sum.
//  * moe_align_kernel    one workgroup per expert: a stable placement of the
//                        rows (t, slot) by (expert, t, slot): a row's
//                        position is offsets[e] (the pairs routed to lower
//                        experts) plus the number of earlier (token, slot)
//                        pairs that chose e (a block-wide scan).
//  * silu_mul_quant_kernel  a = bf16(silu(gate) * up), then the dynamic
//                        per-(row, 128-group) quantisation of a, in one pass
//                        (codes identical to quant_act applied to a).
//  * moe_combine_kernel  out[t] = bf16(sum_s w[t, s] * y2[row_of[t, s]]).
#include "common.hpp"
#include "internal.hpp"

namespace bi8 {

namespace {

constexpr int kAlignThreads = 1024;
constexpr int kMaxExperts = 1024;

// EMAX > 0 (E <= EMAX): the token's logits are loaded into registers at
// once, all loads in flight together; EMAX == 0: read from memory as used.
// Either way the same operations in the same order.
template <int EMAX>
__global__ __launch_bounds__(256) void moe_topk_kernel(const float *__restrict__ logits, int64_t T, int32_t E,
                                                       int32_t k, int32_t renorm, int32_t *__restrict__ ids,
                                                       float *__restrict__ weights) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const float *l = logits + t * E;
    constexpr int kReg = EMAX > 0 ? EMAX : 1;
    float lg[kReg];
    if constexpr (EMAX > 0) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) lg[e] = e < E ? l[e] : -INFINITY;
    }
    auto L = [&](int e) __attribute__((always_inline)) { return EMAX > 0 ? lg[e] : l[e]; };
    constexpr int kLoop = EMAX > 0 ? EMAX : 0x7FFFFFFF;   // e < E is checked as well
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kLoop && e < E; ++e) mx = fmaxf(mx, L(e));
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < kLoop && e < E; ++e) sum += expf(L(e) - mx);
    // pick k times: the largest logit not yet taken (strict >, so ties go to
    // the lower index); "taken" is kept as the list of chosen ids
    int32_t chosen[8];
    float wsum = 0.0f;
    float wv[8];
    for (int j = 0; j < k; ++j) {
        int best = -1;
        float bl = 0.0f;
#pragma unroll
        for (int e = 0; e < kLoop && e < E; ++e) {
            bool taken = false;
            for (int i = 0; i < j; ++i) taken |= chosen[i] == e;
            if (!taken && (best < 0 || L(e) > bl)) {
                best = e;
                bl = L(e);
            }
        }
        chosen[j] = best;
        wv[j] = expf(bl - mx) / sum;
        wsum += wv[j];
    }
    for (int j = 0; j < k; ++j) {
        ids[t * k + j] = chosen[j];
        weights[t * k + j] = renorm ? wv[j] / wsum : wv[j];
    }
}

// One workgroup per expert e.  Rows are ordered by (expert, token, slot), so
// expert e's rows start at the number of (token, slot) pairs routed to a
// lower expert, and a row's place among e's rows is the number of pairs
// routed to e at earlier (token, slot).  Thread i owns Q consecutive tokens
// of each round of kAlignThreads * Q tokens (their K ids are contiguous):
// pass 1 counts the pairs below e over all tokens (a block sum), pass 2
// places e's rows with a block-wide exclusive scan of the per-thread counts.
// ids outside [0, E) count nowhere and get no row.  The last workgroup also
// writes offsets[E].
constexpr int kAlignWaves = kAlignThreads / 64;

// Inclusive prefix sum over the 64 lanes by DPP: shifts right by 1, 2, 4, 8
// within each row of 16 lanes (lanes shifted in from outside the row add 0),
// then lane 15 of rows 0 and 2 added to rows 1 and 3, then lane 31 to rows 2
// and 3.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Block-wide exclusive prefix (thread order) and total of x.  Two barriers;
// wsum is reused.
__device__ __forceinline__ void block_scan(int32_t x, int32_t &before, int32_t &total, int32_t *wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t incl = wave_incl_scan(x);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
        const int32_t c = wsum[w];
        pre += w < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    before = pre + incl - x;
    total = tot;
}

// A round holds at most kAlignThreads * 8 pairs, so the counts of pairs to e
// (low 16 bits) and below e (high 16 bits) travel packed in one word.
template <int K>
__global__ __launch_bounds__(kAlignThreads) void moe_align_kernel(const int32_t *__restrict__ ids, int64_t T,
                                                                  int32_t E, int32_t *__restrict__ sorted_token,
                                                                  int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ row_of) {
    constexpr int Q = K >= 8 ? 1 : 8 / K;   // tokens per thread and round
    constexpr int N = Q * K;
    static_assert(kAlignThreads * N < 65536, "packed counts");
    __shared__ int32_t wsum[kAlignWaves];
    const int32_t e = (int32_t)blockIdx.x;
    const int64_t TK = T * K, round = (int64_t)kAlignThreads * Q;
    // the thread's N ids of the round from r0 (-1 past the end); every load
    // is issued (clamped into range) before any is used
    auto load = [&](int32_t (&v)[N], int64_t r0) __attribute__((always_inline)) {
        const int64_t i0 = (r0 + (int64_t)threadIdx.x * Q) * K;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int64_t i = i0 + j;
            const int32_t x = ids[i < TK ? i : TK - 1];
            v[j] = i < TK ? x : -1;
        }
    };
    auto counts = [&](const int32_t (&v)[N]) __attribute__((always_inline)) {
        int32_t c = 0;
#pragma unroll
        for (int j = 0; j < N; ++j) c += (v[j] == e ? 1 : 0) + (v[j] >= 0 && v[j] < e ? 0x10000 : 0);
        return c;
    };
    // rows of e among v from row r on, in (token, slot) order
    auto place = [&](const int32_t (&v)[N], int64_t r0, int32_t r) __attribute__((always_inline)) {
        const int64_t t0 = r0 + (int64_t)threadIdx.x * Q;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (v[j] == e) {
                const int64_t t = t0 + j / K;
                sorted_token[r] = (int32_t)t;
                row_of[t * K + j % K] = r;
                ++r;
            }
        }
    };
    auto write_offsets = [&](int32_t below, int32_t mine) __attribute__((always_inline)) {
        if (threadIdx.x == 0) {
            offsets[e] = below;
            if (e == E - 1) offsets[E] = below + mine;
        }
    };

    if (T <= round) {   // one round: one load, one scan
        int32_t v[N];
        if (T > 0) load(v, 0);
        else
#pragma unroll
            for (int j = 0; j < N; ++j) v[j] = -1;
        int32_t before, tot;
        block_scan(counts(v), before, tot, wsum);
        write_offsets(tot >> 16, tot & 0xFFFF);
        place(v, 0, (tot >> 16) + (before & 0xFFFF));
        return;
    }
    int32_t below = 0, mine = 0;   // pairs routed below e / to e, over all tokens
    for (int64_t r0 = 0; r0 < T; r0 += round) {
        int32_t v[N];
        load(v, r0);
        int32_t before, tot;
        block_scan(counts(v), before, tot, wsum);
        below += tot >> 16;
        mine += tot & 0xFFFF;
    }
    write_offsets(below, mine);
    int32_t pos = below;
    for (int64_t r0 = 0; r0 < T; r0 += round) {
        int32_t v[N];
        load(v, r0);
        int32_t before, tot;
        block_scan(counts(v) & 0xFFFF, before, tot, wsum);
        place(v, r0, pos + before);
        pos += tot;
    }
}

// One wave covers eight 128-groups of one row in two halves of four; 16 lanes
// per group, 8 entries per lane and half, all four 16-byte loads (gate and up
// of both halves) in flight before any is used.  h row r: gate h[r, i], up
// h[r, I + i].
constexpr int kSiluWaves = 4;
constexpr int kSiluChunks = 2;
__global__ __launch_bounds__(kSiluWaves * 64) void silu_mul_quant_kernel(
    const uint16_t *__restrict__ h, int64_t I, int8_t *__restrict__ aq, float *__restrict__ as,
    uint16_t *__restrict__ a_out, int64_t IB, int64_t waves_per_row, int64_t total_waves) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kSiluWaves + (threadIdx.x >> 6);
    if (wave >= total_waves) return;
    const int64_t r = wave / waves_per_row;
    const int64_t g0 = (wave - r * waves_per_row) * 4 * kSiluChunks + (lane >> 4);
    u32x4 gv[kSiluChunks], uv[kSiluChunks];
#pragma unroll
    for (int c = 0; c < kSiluChunks; ++c) {
        const int64_t g = g0 + 4 * c, i = g * kBlock + (lane & 15) * 8;
        gv[c] = u32x4{0u, 0u, 0u, 0u};
        uv[c] = u32x4{0u, 0u, 0u, 0u};
        if (g < IB && i < I) {   // I % 16 == 0: a lane's 8 entries are all in or all out
            gv[c] = *reinterpret_cast<const u32x4 *>(h + r * 2 * I + i);
            uv[c] = *reinterpret_cast<const u32x4 *>(h + r * 2 * I + I + i);
        }
    }
#pragma unroll
    for (int c = 0; c < kSiluChunks; ++c) {
        const int64_t g = g0 + 4 * c, i = g * kBlock + (lane & 15) * 8;
        const bool valid = g < IB && i < I;
        float a[8];
        uint32_t ab2[4];   // the bf16 activation, two per word
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float s0 = silu_times(bf16_bits_to_f32(gv[c][j] & 0xFFFFu), bf16_bits_to_f32(uv[c][j] & 0xFFFFu));
            const float s1 = silu_times(bf16_bits_to_f32(gv[c][j] >> 16), bf16_bits_to_f32(uv[c][j] >> 16));
            ab2[j] = f32x2_to_bf16x2_bits(s0, s1);
            a[2 * j] = bf16_bits_to_f32(ab2[j] & 0xFFFFu);
            a[2 * j + 1] = bf16_bits_to_f32(ab2[j] >> 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(a[j]));
        amax = group_max16(amax);
        const float s = amax / 127.0f;
        if (!valid) continue;
        uint32_t lo = 0u, hi = 0u;
        if (s != 0.0f) {
            const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= ((uint32_t)quant_code(a[j], s, rs) & 0xFFu) << (8 * j);
                hi |= ((uint32_t)quant_code(a[4 + j], s, rs) & 0xFFu) << (8 * j);
            }
        }
        *reinterpret_cast<uint2 *>(aq + r * I + i) = make_uint2(lo, hi);
        if ((lane & 15) == 0) as[r * IB + g] = s;
        if (a_out) {
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = ab2[j];
            *reinterpret_cast<u32x4 *>(a_out + r * I + i) = o;
        }
    }
}

// One thread per 8 columns of one token.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ y2, int64_t R,
                                                          const int32_t *__restrict__ row_of,
                                                          const float *__restrict__ w, int64_t T, int32_t k,
                                                          int64_t H, uint16_t *__restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = H / 8;
    if (idx >= T * per_row) return;
    const int64_t t = idx / per_row, c = (idx - t * per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < k; ++s) {
        const int32_t r = row_of[t * k + s];
        if (r < 0 || r >= R) continue;   // a row the dispatch never produced contributes nothing
        const float ws = w[t * k + s];
        const u32x4 v = *reinterpret_cast<const u32x4 *>(y2 + r * H + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = (j & 1) ? (v[j >> 1] >> 16) : (v[j >> 1] & 0xFFFFu);
            acc[j] = fmaf(ws, bf16_bits_to_f32(b), acc[j]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_bits(acc[2 * j]) | (f32_to_bf16_bits(acc[2 * j + 1]) << 16);
    *reinterpret_cast<u32x4 *>(out + t * H + c) = o;
}

}  // namespace

hipError_t launch_moe_route(const float *logits, int64_t T, int32_t E, int32_t k, int32_t renorm,
                            int32_t *ids, float *weights, int32_t *sorted_token, int32_t *offsets,
                            int32_t *row_of, hipStream_t stream) {
    if (E > kMaxExperts || k > 8) return hipErrorInvalidValue;
    if (T > 0) {
        const int64_t blocks = (T + 255) / 256;
        if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
        if (E <= 16)
            hipLaunchKernelGGL(moe_topk_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, stream, logits, T, E, k,
                               renorm, ids, weights);
        else
            hipLaunchKernelGGL(moe_topk_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, logits, T, E, k,
                               renorm, ids, weights);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    switch (k) {
#define BI8_ALIGN_CASE(KK)                                                                                    \
    case KK:                                                                                                 \
        hipLaunchKernelGGL(moe_align_kernel<KK>, dim3((unsigned)E), dim3(kAlignThreads), 0, stream, ids, T, E, \
                           sorted_token, offsets, row_of);                                                   \
        break;
        BI8_ALIGN_CASE(1)
        BI8_ALIGN_CASE(2)
        BI8_ALIGN_CASE(3)
        BI8_ALIGN_CASE(4)
        BI8_ALIGN_CASE(5)
        BI8_ALIGN_CASE(6)
        BI8_ALIGN_CASE(7)
        BI8_ALIGN_CASE(8)
#undef BI8_ALIGN_CASE
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t *h, int64_t R, int64_t I, int8_t *aq, float *as,
                                 uint16_t *a_out, hipStream_t stream) {
    const int64_t IB = (I + kBlock - 1) / kBlock;
    const int64_t waves_per_row = (IB + 4 * kSiluChunks - 1) / (4 * kSiluChunks);
    const int64_t total_waves = R * waves_per_row;
    const int64_t blocks = (total_waves + kSiluWaves - 1) / kSiluWaves;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(silu_mul_quant_kernel, dim3((unsigned)blocks), dim3(kSiluWaves * 64), 0, stream, h, I,
                       aq, as, a_out, IB, waves_per_row, total_waves);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t *y2, int64_t R, const int32_t *row_of, const float *w,
                              int64_t T, int32_t k, int64_t H, uint16_t *out, hipStream_t stream) {
    const int64_t threads = T * (H / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y2, R, row_of, w, T, k,
                       H, out);
    return hipGetLastError();
}

}  // namespace bi8
