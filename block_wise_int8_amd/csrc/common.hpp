// Device-side helpers shared by the block-wise INT8 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi8 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define BI8_LDS __attribute__((address_space(3)))
#define BI8_CONST __attribute__((address_space(4)))

// The [128, 128] block this library implements.
constexpr int kBlock = 128;

// Offset that lies beyond every buffer's num_records: a buffer load with it
// returns zero without touching memory.
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (IEEE-754 roundTiesToEven on the
// 16 dropped bits); NaN becomes the canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 values to packed bf16 bits (lo in bits 0..15) by the hardware
// conversion: round to nearest even, as f32_to_bf16_bits, except that a NaN
// keeps an unspecified quiet-NaN pattern.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Exact int32 -> fp32 of an MFMA block sum without a conversion instruction.
// A block sum of 128 int8 x int8 products has |d| <= 128^3 = 2^21 < 2^22.
// The MFMA accumulates it onto kAccBiasBits, the bit pattern of 1.5 * 2^23:
// for |d| < 2^22 the pattern kAccBiasBits + d is the float 1.5 * 2^23 + d
// (the exponent field stays that of 2^23 and the mantissa field, 2^22 + d,
// stays inside [0, 2^23)), and subtracting 1.5 * 2^23 from it is exact
// (both lie within a factor of two of each other), which leaves exactly
// float(d).  One v_sub_f32 replaces a v_cvt_f32_i32, which issues slower
// (measured: about 6 cycles per wave64 instruction against 4).  Kernels take
// `bias` (= kAccBias) from their arguments, so that it sits in a scalar
// register: a subtraction with the 32-bit literal in the instruction
// instead issues slower than the conversion.
constexpr int32_t kAccBiasBits = 0x4B400000;
constexpr float kAccBias = 12582912.0f;   // 1.5 * 2^23

__device__ __forceinline__ float biased_acc_to_f32(int32_t r, float bias) { return __int_as_float(r) - bias; }

// One int8 code clamp(rne(x / s), -127, 127) with x / s the IEEE correctly
// rounded quotient, computed from r = rcp(s), the hardware reciprocal (within
// 1 ulp of 1 / s), by a single multiply.  y = x * r is then within
// |x / s| * 2^-22 <= 3.1e-5 of fl(x / s) for |x / s| <= 127.5, so the two
// round to the same integer unless y lies within 2^-14 of a half-integer;
// those products (and non-finite ones, e.g. r = inf for a subnormal s) take
// the division.
__device__ __forceinline__ int32_t quant_code(float x, float s, float r) {
    const float y = x * r;
    float q = rintf(y);
    if (!(fabsf(y - q) < 0.5f - 0x1p-14f)) q = rintf(x / s);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int32_t)q;
}

// v from the lane n places lower in its row of 16 lanes, cyclically (DPP
// row_ror:n, a register-to-register move; n in 1..15).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(N >= 1 && N <= 15, "row_ror range");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Max over the 16 lanes of an aligned lane group (a row of the wave): after
// rotations by 1, 2, 4 and 8 every lane holds the max of a cyclic window of
// 16, i.e. of the whole row.  Every lane of the wave must execute it.
__device__ __forceinline__ float group_max16(float v) {
    v = fmaxf(v, row_ror<1>(v));
    v = fmaxf(v, row_ror<2>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<8>(v));
    return v;
}

// One group of 128 activations spread over 16 lanes (8 bf16 per lane, in v):
// the group scale s = amax / 127 (IEEE division) and the lane's 8 codes
// (bytes of lo, hi in element order; all zero when s == 0).  Every lane of
// the wave must execute it.
__device__ __forceinline__ float quant_group16(const u32x4 &v, uint32_t &lo, uint32_t &hi) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = group_max16(amax);
    const float s = amax / 127.0f;
    lo = 0u;
    hi = 0u;
    if (s != 0.0f) {
        const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= ((uint32_t)quant_code(f[i], s, r) & 0xFFu) << (8 * i);
            hi |= ((uint32_t)quant_code(f[4 + i], s, r) & 0xFFu) << (8 * i);
        }
    }
    return s;
}

// The 8 bf16 values p[0..8) as one 16-byte chunk, of which only the first n
// are read (values past them are zero: the end of a row); p need only be
// 2-byte aligned.  One 16-byte load when the chunk is whole and aligned,
// else 2-byte loads.
__device__ __forceinline__ u32x4 load_bf16x8_any(const uint16_t *p, int64_t n) {
    if (n >= 8 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) return *reinterpret_cast<const u32x4 *>(p);
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < n) v[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
    return v;
}

// Store the first n (1..8) of the 8 int8 codes in (lo, hi) at dst, with one
// 8-byte store when all 8 are wanted and dst is 8-byte aligned, else byte by
// byte (rows of a K that is not a multiple of 8 start at any byte).
__device__ __forceinline__ void store_codes8(int8_t *dst, uint32_t lo, uint32_t hi, int64_t n) {
    if (n >= 8 && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
        return;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < n) dst[j] = (int8_t)(((j < 4 ? lo : hi) >> (8 * (j & 3))) & 0xFFu);
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

// Raw buffer resource over [base, base + num_bytes): loads at offsets past the
// end return zero (gfx9 raw-buffer range check, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint32_t clamp_bytes(int64_t n) {
    return n <= 0 ? 0u : (n >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)n);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that is also a compiler memory barrier but does not make
// the compiler drain outstanding global loads first (the LDS fills issued by
// buffer-to-LDS loads are waited for explicitly with wait_vmcnt).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace bi8
