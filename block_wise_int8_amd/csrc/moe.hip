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
//  * moe_align_kernel    one workgroup: expert histogram, offsets, then a
//                        stable placement of the rows (t, slot) by (expert,
//                        t): within an expert the rows keep token order, so
//                        a row's position is offsets[e] plus the number of
//                        earlier tokens that chose e (a block-wide ballot
//                        prefix count per expert and chunk of 1024 tokens).
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

__global__ __launch_bounds__(256) void moe_topk_kernel(const float *__restrict__ logits, int64_t T, int32_t E,
                                                       int32_t k, int32_t renorm, int32_t *__restrict__ ids,
                                                       float *__restrict__ weights) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const float *l = logits + t * E;
    float mx = -INFINITY;
    for (int e = 0; e < E; ++e) mx = fmaxf(mx, l[e]);
    float sum = 0.0f;
    for (int e = 0; e < E; ++e) sum += expf(l[e] - mx);
    // pick k times: the largest logit not yet taken (strict >, so ties go to
    // the lower index); "taken" is kept as the list of chosen ids
    int32_t chosen[8];
    float wsum = 0.0f;
    float wv[8];
    for (int j = 0; j < k; ++j) {
        int best = -1;
        float bl = 0.0f;
        for (int e = 0; e < E; ++e) {
            bool taken = false;
            for (int i = 0; i < j; ++i) taken |= chosen[i] == e;
            if (!taken && (best < 0 || l[e] > bl)) {
                best = e;
                bl = l[e];
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

__global__ __launch_bounds__(kAlignThreads) void moe_align_kernel(const int32_t *__restrict__ ids, int64_t T,
                                                                  int32_t E, int32_t k,
                                                                  int32_t *__restrict__ sorted_token,
                                                                  int32_t *__restrict__ offsets,
                                                                  int32_t *__restrict__ row_of) {
    __shared__ int32_t base[kMaxExperts + 1];
    __shared__ int32_t wave_tot[kAlignThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e <= E; e += kAlignThreads) base[e] = 0;
    __syncthreads();
    // histogram (ids outside [0, E) are not counted and get no row)
    for (int64_t i = tid; i < T * k; i += kAlignThreads) {
        const int32_t e = ids[i];
        if (e >= 0 && e < E) atomicAdd(&base[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0;
        for (int e = 0; e < E; ++e) {
            const int32_t c = base[e];
            base[e] = run;
            offsets[e] = run;
            run += c;
        }
        offsets[E] = run;
    }
    __syncthreads();
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t c0 = 0; c0 < T; c0 += kAlignThreads) {
        const int64_t t = c0 + tid;
        const bool valid = t < T;
        int32_t my[8];
        for (int j = 0; j < k; ++j) my[j] = valid ? ids[t * k + j] : -1;
        for (int e = 0; e < E; ++e) {
            int slot = -1;
            for (int j = 0; j < k; ++j)
                if (my[j] == e) slot = j;
            const uint64_t m = __ballot(slot >= 0);
            if (lane == 0) wave_tot[wave] = __popcll(m);
            __syncthreads();
            // every thread reads the wave counts now, before the barrier below:
            // after it the next round overwrites them
            int32_t pre = 0, tot = 0;
            for (int w = 0; w < kAlignThreads / 64; ++w) {
                const int32_t c = wave_tot[w];
                pre += w < wave ? c : 0;
                tot += c;
            }
            if (slot >= 0) {
                const int32_t pos = base[e] + pre + __popcll(m & below);
                sorted_token[pos] = (int32_t)t;
                row_of[t * k + slot] = pos;
            }
            __syncthreads();
            if (tid == 0) base[e] += tot;
        }
    }
}

// silu(g) * u = g / (1 + exp(-g)) * u in fp32, with exp(-g) as the hardware
// 2^x of -g log2(e) (the rounded argument, |g log2(e)| <= 116 here, moves it
// by at most 116 * 2^-24 * ln 2 ~ 5e-6 relative; 2^x itself within 1 ulp) and
// the quotient through the hardware reciprocal (within 1 ulp).  The bf16
// result then differs from a correctly rounded evaluation's only where the
// fp32 value sits within ~1e-5 of a bf16 rounding boundary.  Below g = -80,
// exp(g) nears the fp32 subnormal range
// (and exp(-g) overflows past g = -88.7, which would give zero where the
// result is still a normal bf16), so there the product is formed as
// g * (2^64 exp(g)) * u * 2^-64 with 2^64 exp(g) = exp2(g log2(e) + 64);
// 1 + exp(g) rounds to 1.
__device__ __forceinline__ float silu_times(float g, float u) {
    if (g >= -80.0f) return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504f)) * u;
    const float t = exp2f(fmaf(g, 1.44269504088896341f, 64.0f));
    return ((g * t) * u) * 0x1p-64f;
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
        hipLaunchKernelGGL(moe_topk_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, logits, T, E, k,
                           renorm, ids, weights);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(moe_align_kernel, dim3(1), dim3(kAlignThreads), 0, stream, ids, T, E, k, sorted_token,
                       offsets, row_of);
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
