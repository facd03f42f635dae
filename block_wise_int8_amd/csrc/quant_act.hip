// Dynamic per-(token, 128-group) activation quantisation, bf16 -> int8 + fp32.
//
// Page "[SGLang] Block-wise INT8" (blog.secrett2633.cloud), section 4: with no
// static input scale, the activation scale is computed at run time per token;
// design rationale item 3: int8 values with fp32 scales.  One scale per
// (token, group of 128 consecutive K entries), s = amax / 127, codes
// clamp(rne(x / s), -127, 127), zero codes for an all-zero group.
//
// HBM-bound single pass: 2 B read + 1 B written per element, 4 B per group.
// Layout on the chip: one wave64 covers 4 consecutive groups of one row (16
// lanes per group, 8 bf16 = one 16-byte load per lane), or, for large
// problems, 8 groups in two halves with both loads in flight before either is
// used.  The group max is reduced across the 16 lanes with cross-lane moves.  The
// scale is an IEEE correctly rounded division and denormals are kept (build
// flags); codes come from one multiply by the hardware reciprocal of s, with
// the division taken wherever the two could round apart (quant_code), so
// codes and scales are bit-exact.
#include "common.hpp"
#include "internal.hpp"

namespace bi8 {

namespace {

constexpr int kQuantWaves = 4;          // waves per workgroup

// rows (gather form, may be null): output row m quantises source row
// rows[m] of x (src_rows rows); an index outside [0, src_rows) reads zeros.
// kChunks: 16-byte loads in flight per lane (1 for small problems, where the
// second chunk's arithmetic would only lengthen the critical path).
// ODD: K % 8 != 0 or rows not 16-byte aligned (ldx % 8 != 0, or x itself):
// a lane's chunk may then cross the end of the row or start anywhere; it is
// read by load_bf16x8_any (values past K read as zero) and its codes stored
// byte by byte where the 8-byte store would be unaligned.
template <int kChunks, bool ODD>
__global__ __launch_bounds__(kQuantWaves * 64) void quant_act_kernel(
    const uint16_t *__restrict__ x, int64_t K, int64_t ldx, int8_t *__restrict__ xq,
    float *__restrict__ xs, int64_t KB, int64_t waves_per_row, int64_t total_waves,
    const int32_t *__restrict__ rows, int64_t src_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kQuantWaves + (threadIdx.x >> 6);
    if (wave >= total_waves) return;
    const int64_t m = wave / waves_per_row;
    const int64_t g0 = (wave - m * waves_per_row) * 4 * kChunks + (lane >> 4);
    const int64_t src = rows ? (int64_t)rows[m] : m;
    const bool src_ok = src >= 0 && src < src_rows;
    // Lane chunk j covers group g0 + 4 j.  With K % 8 == 0 a lane's 8
    // elements are either all inside the row or all outside; outside lanes
    // contribute zeros, which change no group max.  Both loads are issued
    // before either is used.
    u32x4 v[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int64_t g = g0 + 4 * j, k = g * kBlock + (lane & 15) * 8;
        v[j] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (ODD) {
            if (g < KB && k < K && src_ok) v[j] = load_bf16x8_any(x + src * ldx + k, K - k);
        } else {
            if (g < KB && k < K && src_ok) v[j] = *reinterpret_cast<const u32x4 *>(x + src * ldx + k);
        }
    }
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int64_t g = g0 + 4 * j, k = g * kBlock + (lane & 15) * 8;
        const bool valid = (g < KB) && (k < K);
        uint32_t lo, hi;
        const float s = quant_group16(v[j], lo, hi);
        if (!valid) continue;
        if constexpr (ODD)
            store_codes8(xq + m * K + k, lo, hi, K - k);
        else
            *reinterpret_cast<uint2 *>(xq + m * K + k) = make_uint2(lo, hi);
        if ((lane & 15) == 0) xs[m * KB + g] = s;
    }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                            float *xs, hipStream_t stream) {
    return launch_quant_act_gather(x, M, ldx, nullptr, M, K, xq, xs, stream);
}

hipError_t launch_quant_act_gather(const uint16_t *x, int64_t src_rows, int64_t ldx, const int32_t *rows,
                                   int64_t M, int64_t K, int8_t *xq, float *xs, hipStream_t stream) {
    const int64_t KB = (K + kBlock - 1) / kBlock;
    const bool odd = K % 8 != 0 || ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0;
    const bool two = !odd && M * KB >= 8192;   // enough groups to fill the chip with two per lane
    const int64_t gpw = two ? 8 : 4;   // groups per wave
    const int64_t waves_per_row = (KB + gpw - 1) / gpw;
    const int64_t total_waves = M * waves_per_row;
    const int64_t blocks = (total_waves + kQuantWaves - 1) / kQuantWaves;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(kQuantWaves * 64);
    if (odd)
        hipLaunchKernelGGL((quant_act_kernel<1, true>), grid, block, 0, stream, x, K, ldx, xq, xs, KB,
                           waves_per_row, total_waves, rows, src_rows);
    else if (two)
        hipLaunchKernelGGL((quant_act_kernel<2, false>), grid, block, 0, stream,
                           x, K, ldx, xq, xs, KB, waves_per_row, total_waves, rows, src_rows);
    else
        hipLaunchKernelGGL((quant_act_kernel<1, false>), grid, block, 0, stream,
                           x, K, ldx, xq, xs, KB, waves_per_row, total_waves, rows, src_rows);
    return hipGetLastError();
}

}  // namespace bi8

// Offline block quantisation of a bf16 weight [N, K] (row stride ldw):
// one scale per 128 x 128 block, s = amax / 127, codes clamp(rne(w / s)).
// Page "[SGLang] Block-wise INT8", sections 1 and 2 (int8-serialised weights
// with one fp32 scale per block) and design rationale item 3.
//
// One workgroup of 256 threads per block: thread t covers row t / 2 of the
// block and its half t % 2 (64 entries, eight 16-byte loads).  The block max
// is reduced over the wave with cross-lane moves, then over the four waves
// through LDS.  Rows past N and 8-entry pieces past K (K % 16 == 0) read as
// zero and are not written.
namespace bi8 {

namespace {

// Max over the 64 lanes of the wave: the row maxima by DPP rotations, then
// the four rows' by lane reads (uniform result).
__device__ __forceinline__ float wave_max64(float v) {
    v = group_max16(v);
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

__global__ __launch_bounds__(256) void quant_weight_kernel(const uint16_t *__restrict__ w, int64_t N, int64_t K,
                                                           int64_t ldw, int8_t *__restrict__ wq,
                                                           float *__restrict__ ws, int64_t KB) {
    __shared__ float wmax[4];
    const int t = threadIdx.x;
    const int64_t bn = blockIdx.y, bk = blockIdx.x;
    const int64_t n = bn * kBlock + (t >> 1);
    const int64_t k0 = bk * kBlock + (t & 1) * 64;
    const bool row_ok = n < N;
    float f[64];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok && k0 + 8 * c < K) v = *reinterpret_cast<const u32x4 *>(w + n * ldw + k0 + 8 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[8 * c + 2 * j] = bf16_bits_to_f32(v[j] & 0xFFFFu);
            f[8 * c + 2 * j + 1] = bf16_bits_to_f32(v[j] >> 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = wave_max64(amax);
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 127.0f;
    const float r = __builtin_amdgcn_rcpf(s);
    if (t == 0) ws[bn * KB + bk] = s;
    if (!row_ok) return;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        if (k0 + 8 * c >= K) break;
        uint32_t lo = 0u, hi = 0u;
        if (s != 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= ((uint32_t)quant_code(f[8 * c + j], s, r) & 0xFFu) << (8 * j);
                hi |= ((uint32_t)quant_code(f[8 * c + 4 + j], s, r) & 0xFFu) << (8 * j);
            }
        }
        *reinterpret_cast<uint2 *>(wq + n * K + k0 + 8 * c) = make_uint2(lo, hi);
    }
}

}  // namespace

hipError_t launch_quant_weight(const uint16_t *w, int64_t N, int64_t K, int64_t ldw, int8_t *wq, float *ws,
                               hipStream_t stream) {
    const int64_t NB = (N + kBlock - 1) / kBlock, KB = (K + kBlock - 1) / kBlock;
    if (NB == 0 || KB == 0) return hipSuccess;
    if (NB > 65535 || KB > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_weight_kernel, dim3((unsigned)KB, (unsigned)NB), dim3(256), 0, stream, w, N, K, ldw,
                       wq, ws, KB);
    return hipGetLastError();
}

}  // namespace bi8

// Per-token quantisation (the per-channel form: one group spanning all K):
// one workgroup of 256 threads per row, two passes over the row (max, then
// codes), 16-byte loads; a row of up to 8192 entries is read once and kept in
// registers for the second pass.  Same arithmetic as the 128-group kernel.
namespace bi8 {

namespace {

// kChunks > 0: the row fits in kChunks 16-byte loads per thread (K <=
// 2048 kChunks), which stay in registers between the two passes; 0: the
// second pass reads the row again.  ODD: K % 8 != 0 or rows not 16-byte
// aligned: chunks read by load_bf16x8_any (values past K read as zero) and
// codes stored byte by byte where the 8-byte store would be unaligned.
template <int kChunks, bool ODD>
__global__ __launch_bounds__(256) void quant_act_token_kernel(const uint16_t *__restrict__ x, int64_t K,
                                                              int64_t ldx, int8_t *__restrict__ xq,
                                                              float *__restrict__ xs) {
    __shared__ float wmax[4];
    const int t = threadIdx.x;
    const int64_t m = blockIdx.x;
    const uint16_t *row = x + m * ldx;
    u32x4 v[kChunks > 0 ? kChunks : 1];
    float amax = 0.0f;
    auto row_max = [&](const u32x4 &c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(c[j] & 0xFFFFu)), fabsf(bf16_bits_to_f32(c[j] >> 16))));
    };
    if constexpr (kChunks > 0) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int64_t k = 8 * (t + 256 * c);
            v[c] = u32x4{0u, 0u, 0u, 0u};
            if (k < K) v[c] = *reinterpret_cast<const u32x4 *>(row + k);
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) row_max(v[c]);
    } else {
        for (int64_t k = 8 * t; k < K; k += 8 * 256)
            row_max(ODD ? load_bf16x8_any(row + k, K - k) : *reinterpret_cast<const u32x4 *>(row + k));
    }
    amax = wave_max64(amax);
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 127.0f;
    const float r = __builtin_amdgcn_rcpf(s);
    if (t == 0) xs[m] = s;
    auto codes = [&](const u32x4 &c, int64_t k) __attribute__((always_inline)) {
        uint32_t lo = 0u, hi = 0u;
        if (s != 0.0f) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lo |= ((uint32_t)quant_code(bf16_bits_to_f32(c[j] & 0xFFFFu), s, r) & 0xFFu) << (16 * j);
                lo |= ((uint32_t)quant_code(bf16_bits_to_f32(c[j] >> 16), s, r) & 0xFFu) << (16 * j + 8);
                hi |= ((uint32_t)quant_code(bf16_bits_to_f32(c[2 + j] & 0xFFFFu), s, r) & 0xFFu) << (16 * j);
                hi |= ((uint32_t)quant_code(bf16_bits_to_f32(c[2 + j] >> 16), s, r) & 0xFFu) << (16 * j + 8);
            }
        }
        if constexpr (ODD)
            store_codes8(xq + m * K + k, lo, hi, K - k);
        else
            *reinterpret_cast<uint2 *>(xq + m * K + k) = make_uint2(lo, hi);
    };
    if constexpr (kChunks > 0) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int64_t k = 8 * (t + 256 * c);
            if (k < K) codes(v[c], k);
        }
    } else {
        for (int64_t k = 8 * t; k < K; k += 8 * 256)
            codes(ODD ? load_bf16x8_any(row + k, K - k) : *reinterpret_cast<const u32x4 *>(row + k), k);
    }
}

}  // namespace

hipError_t launch_quant_act_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *xq,
                                      float *xs, hipStream_t stream) {
    if (M == 0) return hipSuccess;
    if (M > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const int64_t chunks = (K + 2047) / 2048;   // 16-byte loads per thread
    const dim3 grid((unsigned)M), block(256);
    if (K % 8 != 0 || ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0)
        hipLaunchKernelGGL((quant_act_token_kernel<0, true>), grid, block, 0, stream, x, K, ldx, xq, xs);
    else if (chunks <= 1)
        hipLaunchKernelGGL((quant_act_token_kernel<1, false>), grid, block, 0, stream, x, K, ldx, xq, xs);
    else if (chunks <= 2)
        hipLaunchKernelGGL((quant_act_token_kernel<2, false>), grid, block, 0, stream, x, K, ldx, xq, xs);
    else if (chunks <= 4)
        hipLaunchKernelGGL((quant_act_token_kernel<4, false>), grid, block, 0, stream, x, K, ldx, xq, xs);
    else
        hipLaunchKernelGGL((quant_act_token_kernel<0, false>), grid, block, 0, stream, x, K, ldx, xq, xs);
    return hipGetLastError();
}

}  // namespace bi8
