// Block-scaled int8 GEMM kernels for gfx950: y = bf16( sum_g acc_g * xs * ws ).
//
// Page "[SGLang] Block-wise INT8" (blog.secrett2633.cloud): structure diagram
// and section 2 (int8 weight [N, K], fp32 scale per 128 x 128 block, scale
// tensor [ceil(N/128), ceil(K/128)]); section 4 (the linear consumes the int8
// weight, its block scales and dynamic per-token activation scales, plus an
// optional bias); section 5/6 (per-expert weights and scales for MoE);
// design rationale item 1 (a 128 x 128 block matches the GEMM tile) and
// item 3 (fp32 scales multiply on dequantisation).
//
// Both kernels put the WEIGHT rows in the MFMA's A operand (rows of the MFMA
// result = output columns n) and the activation rows in the B operand
// (columns of the result = tokens m).  A lane of the 32x32 (16x16) result then
// holds a single token and 16 (4) output columns that all sit in one 128-row
// weight block, so the per-block rescale needs ONE fp32 factor per lane:
// t = xs[m, g] * ws[n / 128, g], applied as y = fma(float(acc_int32), t, y).
//
// Paths:
//  * skinny (decode; M <= 64 with N small enough): HBM streaming of W.  A
//    workgroup owns 16 weight rows; its 8 waves split K.  Each lane loads 32 contiguous bytes of
//    one weight row per 128-block straight into registers (no LDS), issues all
//    of its loads before the first MFMA (v_mfma_i32_16x16x64_i8), and the
//    waves' fp32 partials are summed through LDS.
//  * tiled (the other shapes: prefill, MoE): int8 MFMA v_mfma_i32_32x32x32_i8.  A
//    workgroup computes a (64*WN) x (64*WM) tile (W rows x X rows), one 64x64
//    sub-tile per wave.  K advances one 128-block per step; both operand tiles
//    are staged in LDS by buffer->LDS loads (no VGPR round trip) through a
//    3-deep ring, one LDS array per stage, rows of 128 B with the 16-byte
//    chunks XOR-swizzled so the MFMA fragment reads are bank-conflict free.
//    The per-block activation scales ride in the same stage.  Out-of-range
//    rows (M, N tails, MoE segment ends) and the K tail read as zero through
//    the buffer range check, which is exactly zero padding.
#include "common.hpp"
#include "internal.hpp"

namespace bi8 {

namespace {

struct GemmArgs {
    const int8_t *xq;
    const float *xs;
    const int8_t *w;
    const float *ws;
    const uint16_t *bias;
    uint16_t *y;
    const int32_t *offsets;   // MoE only: [E + 1] row offsets per expert
    int64_t M;                // rows (R for MoE)
    int64_t N;
    int64_t K;
    int64_t KB;               // ceil(K / 128)
    int64_t NB;               // ceil(N / 128)
    int64_t tiles_m;          // dense: ceil(M / BM); MoE: upper bound of m-tiles
    int64_t tiles_n;
    int32_t E;
    int32_t wide_store;       // y rows allow 8-byte stores (N % 4 == 0, y 8-byte aligned)
};

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

__device__ __forceinline__ i32x4 as_i32x4(u32x4 v) {
    return __builtin_bit_cast(i32x4, v);
}

// ---------------------------------------------------------------------------
// Skinny path (M <= 64)
// ---------------------------------------------------------------------------

constexpr int kSkinnyWaves = 8;
constexpr int64_t kSkinnyMaxM = 64;
// Crossovers at K = 4096 (skinny / tiled, us): block form M = 24, N = 8192:
// 17.4 / 18.6, M = 32, N = 8192: 19.6 / 18.8, M = 8, N = 28672: 31.0 / 27.0;
// per-channel M = 16, N = 28672: 32.0 / 37.0, M = 24, N = 28672: 38.2 / 35.4.
constexpr int64_t kSkinnyBudget = 360000;     // block form
constexpr int64_t kSkinnyBudgetPC = 1024000;  // per-channel form
constexpr int kSkinnyUnroll = 4;

// MT: 16-token column tiles (1 to 4: M <= 16, 32, 48, 64).  PC: the
// per-channel form (blocks of 1 x K): the block sums are added unscaled and
// the token and weight-row scales multiply once, in the store.
template <int MT, bool PC>
__global__ __launch_bounds__(kSkinnyWaves * 64) void gemm_skinny_kernel(GemmArgs p,
                                                                       int32_t blocks_per_wave) {
    // loads of U K blocks are in flight per wave (fewer with 4 token tiles:
    // the activation operands take registers too)
    constexpr int U = MT <= 3 ? kSkinnyUnroll : 2;
    __shared__ float red[kSkinnyWaves][MT][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane & 15;    // weight row in the tile, and token column
    const int quad = lane >> 4;   // 32-byte quarter of a 128-wide K block
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t K = p.K, KB = p.KB;

    // Each range covers only what this workgroup may read (<= 2^31 bytes since
    // K <= 2^23), so kOobOffset always lies past it.
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(p.w + n0 * K, clamp_bytes((p.N - n0 < 16 ? p.N - n0 : 16) * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq, clamp_bytes(p.M * K));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.xs, clamp_bytes(p.M * KB * 4));
    const float *ws_row = p.ws + (n0 / kBlock) * KB;

    const int64_t b_begin = (int64_t)wave * blocks_per_wave;
    const int64_t b_end = b_begin + blocks_per_wave < KB ? b_begin + blocks_per_wave : KB;

    f32x4 yv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) yv[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t b0 = b_begin; b0 < b_end; b0 += U) {
        i32x4 wa[U][2];
        i32x4 xb[U][MT][2];
        float xsv[U][MT];
        float wsv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t b = b0 + u;
            const bool ok = b < b_end;
            const int64_t kk = b * kBlock + quad * 32;
            const bool in0 = ok && kk < K, in1 = ok && kk + 16 < K;
            wa[u][0] = as_i32x4(buf_load16(wr, in0 ? (uint32_t)(row * K + kk) : kOobOffset));
            wa[u][1] = as_i32x4(buf_load16(wr, in1 ? (uint32_t)(row * K + kk + 16) : kOobOffset));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // lanes of token columns past M load nothing (zero operands)
                const int64_t tok = mt * 16 + row;
                xb[u][mt][0] = i32x4{0, 0, 0, 0};
                xb[u][mt][1] = i32x4{0, 0, 0, 0};
                if constexpr (!PC) xsv[u][mt] = 0.f;
                if (tok < p.M) {
                    xb[u][mt][0] = as_i32x4(buf_load16(xr, in0 ? (uint32_t)(tok * K + kk) : kOobOffset));
                    xb[u][mt][1] =
                        as_i32x4(buf_load16(xr, in1 ? (uint32_t)(tok * K + kk + 16) : kOobOffset));
                    if constexpr (!PC)
                        xsv[u][mt] = buf_load_f32(sr, ok ? (uint32_t)((tok * KB + b) * 4) : kOobOffset);
                }
            }
            if constexpr (!PC) wsv[u] = ws_row[ok ? b : KB - 1];
        }
        // every load above is issued before the first MFMA: without this the
        // scheduler interleaves loads and MFMAs and the wave pays several HBM
        // round trips instead of one
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][0], xb[u][mt][0],
                                                                  i32x4{0, 0, 0, 0}, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][1], xb[u][mt][1], acc, 0, 0, 0);
                if constexpr (PC) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) yv[mt][i] += (float)acc[i];
                } else {
                    const float t = xsv[u][mt] * wsv[u];
#pragma unroll
                    for (int i = 0; i < 4; ++i) yv[mt][i] = fmaf((float)acc[i], t, yv[mt][i]);
                }
            }
        }
    }

    // 16x16 result layout: lane -> token column (lane & 15), weight rows
    // 4 * (lane >> 4) + i.  Sum the waves' partials through LDS.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][mt][lane][i] = yv[mt][i];
    __syncthreads();
    for (int t = threadIdx.x; t < MT * 256; t += kSkinnyWaves * 64) {
        const int mt = t >> 8, c = (t >> 4) & 15, r = t & 15;
        const int src = c + 16 * (r >> 2), i = r & 3;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < kSkinnyWaves; ++v) s += red[v][mt][src][i];
        const int64_t tok = mt * 16 + c, n = n0 + r;
        if (tok < p.M && n < p.N) {
            if constexpr (PC) s *= p.xs[tok] * p.ws[n];
            if (p.bias) s += bf16_bits_to_f32(p.bias[n]);
            p.y[tok * p.N + n] = (uint16_t)f32_to_bf16_bits(s);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled path
// ---------------------------------------------------------------------------

// WN x WM waves per workgroup; each wave owns SA x SB sub-tiles of 32 x 32
// (weight rows x activation rows).
template <int WN, int WM, int SA, int SB>
struct TileCfg {
    static constexpr int kWaves = WN * WM;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kWaveN = 32 * SA;           // weight rows per wave
    static constexpr int kWaveM = 32 * SB;           // activation rows per wave
    static constexpr int kBN = kWaveN * WN;          // weight rows per tile
    static constexpr int kBM = kWaveM * WM;          // activation rows per tile
    static constexpr int kWOff = 0;                  // LDS layout of one stage
    static constexpr int kXOff = kBN * 128;
    static constexpr int kStageBytes = kXOff + kBM * 128;
    static constexpr int kWLoads = kBN / 8 / kWaves; // 1 KB W pieces per wave per stage
    static constexpr int kXLoads = kBM / 8 / kWaves; // 1 KB X pieces per wave per stage
    static constexpr int kTileLoads = kWLoads + kXLoads;
    // Activation scales travel in batches of kSB K blocks: one 32-byte run per
    // tile row and batch (one memory line) instead of one 4-byte gather per
    // row and block.  kScaleLoads dword loads per wave carry one batch.
    static constexpr int kSB = 8;
    static constexpr int kScaleLoads = kBM * kSB / 64 / kWaves;
    static_assert(kWLoads >= 1 && kXLoads >= 1 && kBN % (8 * kWaves) == 0 && kBM % (8 * kWaves) == 0,
                  "load split");
    static_assert(128 % kWaveN == 0, "a wave's weight rows lie in one 128-row scale block");
    static_assert(kScaleLoads >= 1 && kBM * kSB % (64 * kWaves) == 0, "scale batch split");
};

// Spread consecutive workgroup ids (dispatched round-robin over the 8 XCDs)
// so that each XCD receives a contiguous range of tiles and its L2 sees
// neighbouring tiles.  Bijective on [0, total).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
    const int64_t q = total >> 3, r = total & 7;
    const int64_t xcd = bid & 7, slot = bid >> 3;
    return xcd * q + (xcd < r ? xcd : r) + slot;
}

// m-tiles per group in the tile order: consecutive workgroups walk a group's
// m-tiles for one n-tile, then the next n-tile (measured: 8 for the 256 x 128
// tile, 4 for 256 x 256, where 8 was 15 % slower at 4096^3)
constexpr int64_t kGroupM = 8;
constexpr int64_t kGroupMWide = 4;

struct Tile {
    int64_t n0;    // first weight row / output column
    int64_t m0;    // first activation row (global row of xq, xs, y)
    int64_t rows;  // valid activation rows in this tile
    const int8_t *w;
    const float *ws;
};

template <int BN, int BM, bool MOE, int64_t GM = kGroupM>
__device__ __forceinline__ bool decode_tile(const GemmArgs &p, Tile &t) {
    const int64_t total = p.tiles_m * p.tiles_n;
    const int64_t tid = xcd_remap(blockIdx.x, total);
    // grouped order: GM m-tiles advance together along n
    const int64_t group = tid / (GM * p.tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsize = p.tiles_m - first_m < GM ? p.tiles_m - first_m : GM;
    const int64_t in = tid - group * GM * p.tiles_n;
    int64_t tm = first_m + in % gsize;
    const int64_t tn = in / gsize;
    t.n0 = tn * BN;
    if constexpr (!MOE) {
        t.m0 = tm * BM;
        t.rows = p.M - t.m0 < BM ? p.M - t.m0 : BM;
        t.w = p.w;
        t.ws = p.ws;
        return true;
    } else {
        for (int32_t e = 0; e < p.E; ++e) {
            // clamp to [0, R] so that offsets breaking the precondition can
            // never address rows outside xq / y
            int64_t a = p.offsets[e], b = p.offsets[e + 1];
            a = a < 0 ? 0 : (a > p.M ? p.M : a);
            b = b < a ? a : (b > p.M ? p.M : b);
            const int64_t cnt = (b - a + BM - 1) / BM;
            if (tm < cnt) {
                t.m0 = a + tm * BM;
                t.rows = b - t.m0 < BM ? b - t.m0 : BM;
                t.w = p.w + (int64_t)e * p.N * p.K;
                t.ws = p.ws + (int64_t)e * p.NB * p.KB;
                return true;
            }
            tm -= cnt;
        }
        return false;
    }
}

// PING: the two wave groups (rows wm = 0 and wm = 1 of the wave grid; waves w
// and w + 4 share a SIMD) run half a K step apart.  Per K step there are two
// barriers; between them one group issues its MFMAs while the other converts
// and rescales its previous block (VALU), so each SIMD keeps its matrix core
// and its vector ALU busy at the same time.
template <int WN, int WM, int SA, int SB, bool MOE, bool PING, int NS>
__global__ __launch_bounds__(WN *WM * 64) void gemm_tiled_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    // (device pass only: the body's address-space casts are not valid host
    // code, and the host pass only needs the launch stub)
    using C = TileCfg<WN, WM, SA, SB>;
    static_assert(!PING || (WM == 2 && WN == 4), "ping-pong pairs waves w and w + 4 on one SIMD");
    // the ring: NS stages, loads NS - 1 blocks ahead; a scale batch (kSB
    // blocks) must be published before the next one's loads are issued
    static_assert(NS >= 3 && NS <= 6 && NS - 2 < C::kSB, "ring depth");
    // one array per stage: with a separate object per stage the compiler
    // knows which in-flight fills a fragment read cannot alias
    __shared__ __attribute__((aligned(1024))) char lds0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds2[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds3[NS > 3 ? C::kStageBytes : 1];
    __shared__ __attribute__((aligned(1024))) char lds4[NS > 4 ? C::kStageBytes : 1];
    __shared__ __attribute__((aligned(1024))) char lds5[NS > 5 ? C::kStageBytes : 1];
    auto lds = [&](const int i) __attribute__((always_inline)) -> char * {
        return i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : i == 3 ? lds3 : i == 4 ? lds4 : lds5;
    };
    __shared__ float xsl[2][C::kBM * C::kSB];   // activation-scale batches, double-buffered

    Tile t;
    if (!decode_tile<C::kBN, C::kBM, MOE>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K, KB = p.KB;

    // Each range covers only this tile's rows (<= 2^31 bytes since K <= 2^23),
    // so kOobOffset always lies past it.
    const int64_t wrows = p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq + t.m0 * K, clamp_bytes(t.rows * K));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.xs + t.m0 * KB, clamp_bytes(t.rows * KB * 4));

    // Per-lane load descriptors.  Load piece q (1 KB) covers tile rows
    // [8q, 8q+8); lane i lands at LDS row 8q + i/8, 16-byte slot i%8, which
    // holds K chunk c = slot ^ swz(row), swz(r) = (r & 7) ^ ((r >> 3) & 1).
    const int r_in = lane >> 3;
    uint32_t wgo[C::kWLoads], xgo[C::kXLoads];   // global offset at kb = 0
    int wchunk[C::kWLoads], xchunk[C::kXLoads];
#pragma unroll
    for (int j = 0; j < C::kWLoads; ++j) {
        const int q = wave + j * C::kWaves;
        const int c = (lane & 7) ^ r_in ^ (q & 1);
        wchunk[j] = 16 * c;
        wgo[j] = (uint32_t)((8 * q + r_in) * K + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < C::kXLoads; ++j) {
        const int q = wave + j * C::kWaves;
        const int c = (lane & 7) ^ r_in ^ (q & 1);
        xchunk[j] = 16 * c;
        xgo[j] = (uint32_t)((8 * q + r_in) * K + 16 * c);
    }
    // Scale batch layout (per buffer): row-major [kBM rows][kSB blocks]; this
    // wave's load j covers flat entries f = (wave * kScaleLoads + j) * 64 + lane.
    float sv[C::kScaleLoads];

    // Issue one stage's buffer->LDS loads for K block kb.  A chunk at or past
    // K (the K tail, and every chunk of a block kb >= KB) reads as zero; the
    // check is a per-lane select with no branch (a branch here makes the
    // compiler lose track of which stage each LDS fill writes and drain the
    // prefetch).  With the first block of a scale batch, the batch's scales
    // are loaded into registers (issued first, so they complete with the
    // stage); they are written to LDS one step before the batch is used.
    auto issue = [&](char *stage, int64_t kb) __attribute__((always_inline)) {
        const int64_t k0 = kb * kBlock;
        const uint32_t kofs = (uint32_t)k0;
        if ((kb & (C::kSB - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < C::kScaleLoads; ++j) {
                const int f = (wave * C::kScaleLoads + j) * 64 + lane;
                const int64_t g = kb + (f & (C::kSB - 1));
                sv[j] = buf_load_f32(sr, g < KB ? (uint32_t)(((f / C::kSB) * KB + g) * 4) : kOobOffset);
            }
        }
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (BI8_LDS void *)(stage + C::kWOff + (wave + j * C::kWaves) * 1024), 16,
                (k0 + wchunk[j] < K) ? wgo[j] + kofs : kOobOffset, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (BI8_LDS void *)(stage + C::kXOff + (wave + j * C::kWaves) * 1024), 16,
                (k0 + xchunk[j] < K) ? xgo[j] + kofs : kOobOffset, 0, 0, 0);
    };
    // Write the scale batch held in registers to LDS buffer `half`, and make it
    // visible before the next barrier.
    auto store_scales = [&](const int64_t half) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < C::kScaleLoads; ++j)
            xsl[half][(wave * C::kScaleLoads + j) * 64 + lane] = sv[j];
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));   // lgkmcnt(0)
    };

    // Fragment read addresses (32x32x32 operand layout: lane -> row lane & 31,
    // 16-byte K chunk 2*s + (lane >> 5) for k-step s).
    const int wn = wave % WN, wm = wave / WN;
    const int rr = lane & 31, hi = lane >> 5;
    const int swz = (rr & 7) ^ ((rr >> 3) & 1);
    int frag_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) frag_off[s] = 16 * ((2 * s + hi) ^ swz);
    const int wrow0 = C::kWOff + (wn * C::kWaveN + rr) * 128;
    const int xrow0 = C::kXOff + (wm * C::kWaveM + rr) * 128;
    int srow[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) srow[b] = (wm * C::kWaveM + 32 * b + rr) * C::kSB;

    int64_t nbw = (t.n0 + wn * C::kWaveN) / kBlock;
    if (nbw > p.NB - 1) nbw = p.NB - 1;
    // The wave's weight-scale row, read through the constant address space so
    // that the wave-uniform loads become scalar loads (the scales are never
    // written while the kernel runs).
    const BI8_CONST float *ws_row = reinterpret_cast<const BI8_CONST float *>(
        reinterpret_cast<uintptr_t>(t.ws + nbw * KB));

    i32x16 zero16;
#pragma unroll
    for (int i = 0; i < 16; ++i) zero16[i] = 0;
    f32x16 y[SA][SB];
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) y[a][b][i] = 0.f;

    // MFMA phase: the block's int32 sums for the wave's 2 x 2 sub-tiles, plus
    // the scales the rescale will need (read now: the stage may be refilled
    // before the rescale runs).
    i32x16 acc[SA][SB];
    float xsv[SB], wsv = 0.f;
    auto mma = [&](const char *stage, int64_t kb) __attribute__((always_inline)) {
        i32x4 wf[SA][4], xf[SB][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int a = 0; a < SA; ++a)
                wf[a][s] = *reinterpret_cast<const i32x4 *>(stage + wrow0 + a * 32 * 128 + frag_off[s]);
#pragma unroll
            for (int b = 0; b < SB; ++b)
                xf[b][s] = *reinterpret_cast<const i32x4 *>(stage + xrow0 + b * 32 * 128 + frag_off[s]);
        }
#pragma unroll
        for (int b = 0; b < SB; ++b)
            xsv[b] = xsl[(kb / C::kSB) & 1][srow[b] + (kb & (C::kSB - 1))];
        wsv = ws_row[kb];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < SA; ++a)
#pragma unroll
                for (int b = 0; b < SB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        wf[a][s], xf[b][s], s == 0 ? zero16 : acc[a][b], 0, 0, 0);
        // the MFMAs belong to this phase
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < SB; ++b) asm volatile("" : "+v"(acc[a][b]));
    };
    // Rescale phase: y += float(acc) * (xs * ws) per sub-tile.
    auto epi = [&]() __attribute__((always_inline)) {
        float tb[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) tb[b] = xsv[b] * wsv;
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < SB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    y[a][b][i] = fmaf((float)acc[a][b][i], tb[b], y[a][b][i]);
        // the rescale belongs to this phase
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < SB; ++b) asm volatile("" : "+v"(y[a][b]));
    };
    // Before step kb, only the loads of blocks kb + 1 .. kb + NS - 2 may still
    // be in flight, plus the scale batch of the one of them that starts a
    // batch (at most one does: NS - 2 < kSB).
    auto wait_stage = [&](int64_t kb) __attribute__((always_inline)) {
        if ((int)(kb & (C::kSB - 1)) >= C::kSB - (NS - 2))
            wait_vmcnt<(NS - 2) * C::kTileLoads + C::kScaleLoads>();
        else
            wait_vmcnt<(NS - 2) * C::kTileLoads>();
    };

    // NS-stage ring: block kb lives in lds[kb % NS]; loads run NS - 1 blocks
    // ahead.  Before the first barrier of step kb, this wave's loads of block
    // kb are complete.
    auto step = [&](const int group, char *cur, char *ahead, int64_t kb) __attribute__((always_inline)) {
        wait_stage(kb);
        lds_barrier();
        issue(ahead, kb + NS - 1);
        if (!PING || group == 0) {
            mma(cur, kb);
            if (PING) lds_barrier();
            epi();
        } else {
            if (kb > 0) epi();   // block kb - 1
            lds_barrier();
            mma(cur, kb);
        }
        // the next block opens a new scale batch: publish it (its loads were
        // issued with block kb + 1's stage, a step ago)
        if (((kb + 1) & (C::kSB - 1)) == 0) store_scales(((kb + 1) / C::kSB) & 1);
    };
    auto run = [&](const int group) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NS - 1; ++i) issue(lds(i), i);
        store_scales(0);
        int64_t kb = 0;
        for (; kb + NS <= KB; kb += NS) {
#pragma unroll
            for (int i = 0; i < NS; ++i) step(group, lds(i), lds((i + NS - 1) % NS), kb + i);
        }
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (kb < KB) step(group, lds(i), lds((i + NS - 1) % NS), kb++);
        if (PING && group == 1) epi();   // the last block
    };
    if (!PING || wm == 0)
        run(0);
    else
        run(1);
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

    // Store.  32x32 result layout: lane -> token column (lane & 31); element i
    // -> weight row 8 * (i / 4) + 4 * (lane >> 5) + (i % 4).
#pragma unroll
    for (int b = 0; b < SB; ++b) {
        const int64_t ml = wm * C::kWaveM + b * 32 + rr;
        if (ml >= t.rows) continue;
        uint16_t *yrow = p.y + (t.m0 + ml) * p.N;
#pragma unroll
        for (int a = 0; a < SA; ++a) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t n = t.n0 + wn * C::kWaveN + a * 32 + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = y[a][b][4 * i4 + e];
                    if (p.bias && n + e < p.N) v[e] += bf16_bits_to_f32(p.bias[n + e]);
                }
                if (p.wide_store) {
                    if (n < p.N) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// Wide tiled path: 256 weight rows x 256 activation rows per workgroup
// ---------------------------------------------------------------------------
//
// Moving a tile's operands from L2 into LDS costs (BN + BM) * 128 bytes per K
// block for BN * BM * 128 MACs, so the 256 x 256 tile moves a third fewer
// bytes per MAC than 256 x 128.  Its 8 waves (a 2 x 4 grid, 128 weight rows x
// 64 activation rows each, i.e. 4 x 2 sub-tiles of 32 x 32) cannot hold a
// whole block's int32 sums next to the fp32 accumulators, so the rescale is
// pipelined per sub-tile instead: while the MFMAs of sub-tile j run, the VALU
// converts and rescales sub-tile j - 1 (two 16-register int32 buffers).  Two
// 64 KB stages form the LDS ring: block kb + 1 is loaded while block kb is
// computed, and the barrier and first fragment reads of block kb + 1 overlap
// the last rescale of block kb.  The activation scales reach LDS by
// buffer-to-LDS loads, eight K blocks at a time, without passing through
// registers.
struct WideCfg {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int WN = 2, WM = 4;      // wave grid
    static constexpr int SA = 4, SB = 2;      // 32 x 32 sub-tiles per wave
    static constexpr int kWaveN = 32 * SA;    // 128 weight rows: one scale block
    static constexpr int kWaveM = 32 * SB;    // 64 activation rows
    static constexpr int kBN = kWaveN * WN;   // 256
    static constexpr int kBM = kWaveM * WM;   // 256
    static constexpr int kXOff = kBN * 128;
    static constexpr int kStageBytes = kXOff + kBM * 128;
    static constexpr int kWLoads = kBN / 8 / kWaves;
    static constexpr int kXLoads = kBM / 8 / kWaves;
    static constexpr int kSB = 8;
    static constexpr int kScaleLoads = kBM * kSB / 64 / kWaves;
};

template <bool MOE>
__global__ __launch_bounds__(WideCfg::kThreads) void gemm_wide_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = WideCfg;
    constexpr int SA = C::SA, SB = C::SB;
    __shared__ __attribute__((aligned(1024))) char lds0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[C::kStageBytes];
    __shared__ float xsl[2][C::kBM * C::kSB];

    Tile t;
    if (!decode_tile<C::kBN, C::kBM, MOE, kGroupMWide>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K, KB = p.KB;

    const int64_t wrows = p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq + t.m0 * K, clamp_bytes(t.rows * K));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.xs + t.m0 * KB, clamp_bytes(t.rows * KB * 4));

    // Load pieces as in the 3-stage kernel: piece q (1 KB) covers tile rows
    // [8q, 8q+8), lane i lands at LDS row 8q + i/8, slot i%8, which holds K
    // chunk slot ^ swz(row).
    // Pieces q = wave + 8 j all have the parity of `wave`, so every piece of
    // a lane uses the same chunk and its offsets differ by j * 64 rows.
    const int r_in = lane >> 3;
    const int chunk = 16 * ((lane & 7) ^ r_in ^ (wave & 1));
    const uint32_t go = (uint32_t)((8 * wave + r_in) * K + chunk);
    const uint32_t piece_stride = (uint32_t)(8 * C::kWaves * K);
    uint32_t sofs[C::kScaleLoads];   // byte offset of this lane's scale entry at kb = 0
#pragma unroll
    for (int j = 0; j < C::kScaleLoads; ++j) {
        const int f = (wave * C::kScaleLoads + j) * 64 + lane;
        sofs[j] = (uint32_t)(((f / C::kSB) * KB + (f & (C::kSB - 1))) * 4);
    }
    // K blocks this lane's 16-byte chunk lies in: kb < kb_in <=> kb * 128 + chunk < K
    const int kb_in = (int)((K - chunk + kBlock - 1) / kBlock);

    auto issue = [&](char *stage, int64_t kb) __attribute__((always_inline)) {
        const uint32_t kofs = (uint32_t)kb * kBlock;
        if ((kb & (C::kSB - 1)) == 0) {
            // The batch of activation scales goes straight to LDS, 4 bytes a
            // lane.  Entries past the last K block read the next row's scales
            // (or zero past the end of xs): they are never used, so no check.
#pragma unroll
            for (int j = 0; j < C::kScaleLoads; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    sr, (BI8_LDS void *)&xsl[(kb / C::kSB) & 1][(wave * C::kScaleLoads + j) * 64], 4,
                    sofs[j] + (uint32_t)kb * 4u, 0, 0, 0);
        }
        const bool in_k = (int)kb < kb_in;
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (BI8_LDS void *)(stage + (wave + j * C::kWaves) * 1024), 16,
                in_k ? go + kofs + j * piece_stride : kOobOffset, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (BI8_LDS void *)(stage + C::kXOff + (wave + j * C::kWaves) * 1024), 16,
                in_k ? go + kofs + j * piece_stride : kOobOffset, 0, 0, 0);
    };

    const int wn = wave % C::WN, wm = wave / C::WN;
    const int rr = lane & 31, hi = lane >> 5;
    const int swz = (rr & 7) ^ ((rr >> 3) & 1);
    int frag_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) frag_off[s] = 16 * ((2 * s + hi) ^ swz);
    const int wrow0 = (wn * C::kWaveN + rr) * 128;
    const int xrow0 = C::kXOff + (wm * C::kWaveM + rr) * 128;
    int srow[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) srow[b] = (wm * C::kWaveM + 32 * b + rr) * C::kSB;

    int64_t nbw = (t.n0 + wn * C::kWaveN) / kBlock;
    if (nbw > p.NB - 1) nbw = p.NB - 1;
    const BI8_CONST float *ws_row = reinterpret_cast<const BI8_CONST float *>(
        reinterpret_cast<uintptr_t>(t.ws + nbw * KB));
    // The weight scale of a block is a scalar load issued one block ahead:
    // scalar loads complete out of order, so a use right after the load would
    // wait for every outstanding LDS read as well.
    float ws_cur = ws_row[0];

    i32x16 zero16;
#pragma unroll
    for (int i = 0; i < 16; ++i) zero16[i] = 0;
    f32x16 y[SA][SB];
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) y[a][b][i] = 0.f;

    auto rescale = [&](const i32x16 &acc, f32x16 &yv, float tb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) yv[i] = fmaf((float)acc[i], tb, yv[i]);
        // a use right here keeps machine sinking from moving the rescales past
        // the next branch (which would keep all accumulators live at once)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(yv[i]));
    };

    // The first fragments of a K block (all activation fragments, the first
    // weight fragments) and its scales.  They are read at the end of the
    // previous block, between its last MFMAs and its last rescale, whose
    // registers they reuse.
    i32x4 xf[SB][4], wf0[4];
    float xsv[SB], wsv;
    auto read_first = [&](const char *stage, int64_t kb) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < SB; ++b) xsv[b] = xsl[(kb / C::kSB) & 1][srow[b] + (kb & (C::kSB - 1))];
#pragma unroll
        for (int s = 0; s < 4; ++s) wf0[s] = *reinterpret_cast<const i32x4 *>(stage + wrow0 + frag_off[s]);
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xf[b][s] = *reinterpret_cast<const i32x4 *>(stage + xrow0 + b * 32 * 128 + frag_off[s]);
        wsv = ws_cur;
        ws_cur = ws_row[kb + 1 < KB ? kb + 1 : KB - 1];   // next block's, issued a block ahead
    };
    // Block kb + 1 is in LDS once this wave's fills have landed and every wave
    // is past the barrier (which also ends every read of block kb): read its
    // first fragments from `nxt`.  After the last block this reads stale LDS
    // that nothing uses.
    auto advance = [&](const char *nxt, int64_t kb) __attribute__((always_inline)) {
        wait_vmcnt<0>();
        lds_barrier();
        read_first(nxt, kb + 1);
    };

    // One K block: first the fills of block kb + 1 into the other stage (its
    // previous block was finished before the last barrier; past the last
    // block they read zeros), then the sub-tiles in the order (a, b) = (0,0),
    // (0,1), (1,0), ...; the rescale of each sub-tile is issued after the next
    // sub-tile's MFMAs, and the last one after the next block's first
    // fragment reads.
    auto compute = [&](const char *stage, char *nxt, int64_t kb) __attribute__((always_inline)) {
        issue(nxt, kb + 1);
        float tb[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) tb[b] = xsv[b] * wsv;
        i32x16 acc[2];
#pragma unroll
        for (int a = 0; a < SA; ++a) {
            i32x4 wf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wf[s] = a == 0 ? wf0[s]
                               : *reinterpret_cast<const i32x4 *>(stage + wrow0 + a * 32 * 128 + frag_off[s]);
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int j = a * SB + b;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[j & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[s], xf[b][s],
                                                                         s == 0 ? zero16 : acc[j & 1], 0, 0, 0);
                if (j > 0) {
                    const int pa = (j - 1) / SB, pb = (j - 1) % SB;
                    rescale(acc[(j - 1) & 1], y[pa][pb], tb[pb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last sub-tile's MFMAs stay ahead of the barrier as well
        asm volatile("" ::"v"(acc[(SA * SB - 1) & 1]));
        advance(nxt, kb);
        rescale(acc[(SA * SB - 1) & 1], y[SA - 1][SB - 1], tb[SB - 1]);
    };

    issue(lds0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    read_first(lds0, 0);
    for (int64_t kb = 0;; kb += 2) {
        // block kb in lds0, block kb + 1 in lds1
        compute(lds0, lds1, kb);
        if (kb + 1 >= KB) break;
        compute(lds1, lds0, kb + 1);
        if (kb + 2 >= KB) break;
    }
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

#pragma unroll
    for (int b = 0; b < SB; ++b) {
        const int64_t ml = wm * C::kWaveM + b * 32 + rr;
        if (ml >= t.rows) continue;
        uint16_t *yrow = p.y + (t.m0 + ml) * p.N;
#pragma unroll
        for (int a = 0; a < SA; ++a) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t n = t.n0 + wn * C::kWaveN + a * 32 + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = y[a][b][4 * i4 + e];
                    if (p.bias && n + e < p.N) v[e] += bf16_bits_to_f32(p.bias[n + e]);
                }
                if (p.wide_store) {
                    if (n < p.N) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// Per-channel path (the degenerate block: block_n = 1, block_k = K)
// ---------------------------------------------------------------------------
//
// One fp32 scale per weight row (ws [N, 1]) and per token (xs [M, 1]): the
// per-channel W8A8 of the SGLang platform matrix ("w8a8_int8") is the block
// form with blocks of 1 x K.  The int32 sums then run over the whole K (no
// per-block rescale; |sum| <= 127^2 K < 2^31 for K <= 2^17) and the fp32
// rescale happens once, in the store: y = float(acc) * xs[m] * ws[n].
// Tiles of 256 weight rows x 128 activation rows, 8 waves of 64 x 64, the
// same 3-stage buffer->LDS ring and swizzle as the block kernel; one barrier
// per K block.
template <bool MOE>
__global__ __launch_bounds__(512) void gemm_perch_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<4, 2, 2, 2>;
    __shared__ __attribute__((aligned(1024))) char lds0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds2[C::kStageBytes];

    Tile t;
    if (!decode_tile<C::kBN, C::kBM, MOE>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K, KB = p.KB;
    const int64_t wrows = p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq + t.m0 * K, clamp_bytes(t.rows * K));

    // pieces q = wave + 8 j share the parity of wave: one chunk per lane
    const int r_in = lane >> 3;
    const int chunk = 16 * ((lane & 7) ^ r_in ^ (wave & 1));
    const uint32_t go = (uint32_t)((8 * wave + r_in) * K + chunk);
    const uint32_t piece_stride = (uint32_t)(8 * C::kWaves * K);
    auto issue = [&](char *stage, int64_t kb) __attribute__((always_inline)) {
        const int64_t k0 = kb * kBlock;
        const bool in_k = k0 + chunk < K;   // also false for every chunk of kb >= KB
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (BI8_LDS void *)(stage + (wave + j * C::kWaves) * 1024),
                                                     16, in_k ? go + (uint32_t)k0 + j * piece_stride : kOobOffset,
                                                     0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (BI8_LDS void *)(stage + C::kXOff + (wave + j * C::kWaves) * 1024), 16,
                in_k ? go + (uint32_t)k0 + j * piece_stride : kOobOffset, 0, 0, 0);
    };

    const int wn = wave % 4, wm = wave / 4;
    const int rr = lane & 31, hi = lane >> 5;
    const int swz = (rr & 7) ^ ((rr >> 3) & 1);
    int frag_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) frag_off[s] = 16 * ((2 * s + hi) ^ swz);
    const int wrow0 = (wn * 64 + rr) * 128;
    const int xrow0 = C::kXOff + (wm * 64 + rr) * 128;

    i32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0;
    auto mma = [&](const char *stage) __attribute__((always_inline)) {
        i32x4 wf[2][4], xf[2][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                wf[a][s] = *reinterpret_cast<const i32x4 *>(stage + wrow0 + a * 32 * 128 + frag_off[s]);
                xf[a][s] = *reinterpret_cast<const i32x4 *>(stage + xrow0 + a * 32 * 128 + frag_off[s]);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[a][s], xf[b][s], acc[a][b], 0, 0, 0);
    };
    // block kb lives in lds[kb % 3]; loads run two blocks ahead
    auto step = [&](char *cur, char *ahead, int64_t kb) __attribute__((always_inline)) {
        wait_vmcnt<C::kTileLoads>();
        lds_barrier();
        issue(ahead, kb + 2);
        mma(cur);
    };
    issue(lds0, 0);
    issue(lds1, 1);
    int64_t kb = 0;
    for (; kb + 3 <= KB; kb += 3) {
        step(lds0, lds2, kb);
        step(lds1, lds0, kb + 1);
        step(lds2, lds1, kb + 2);
    }
    if (kb < KB) step(lds0, lds2, kb++);
    if (kb < KB) step(lds1, lds0, kb++);
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

    // Store: lane -> token column rr; element i -> weight row 8 (i / 4) + 4 hi + i % 4.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t ml = wm * 64 + b * 32 + rr;
        if (ml >= t.rows) continue;
        const float xsv = p.xs[t.m0 + ml];
        uint16_t *yrow = p.y + (t.m0 + ml) * p.N;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t n = t.n0 + wn * 64 + a * 32 + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float wsv = n + e < p.N ? t.ws[n + e] : 0.0f;
                    v[e] = (float)acc[a][b][4 * i4 + e] * (xsv * wsv);
                    if (p.bias && n + e < p.N) v[e] += bf16_bits_to_f32(p.bias[n + e]);
                }
                if (p.wide_store) {
                    if (n < p.N) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Per-channel, 256 x 256 tiles: the wide kernel's tile, wave grid (8 waves of
// 128 weight rows x 64 activation rows), 2-stage LDS ring and swizzle, with no
// per-block scale at all.  Each of a wave's 8 sub-tiles keeps one int32
// accumulator over the whole of K (8 x 16 registers), so a K block is just
// its fragment reads and 32 MFMAs; the fp32 scales multiply once, in the
// store.  For problems with enough 256 x 256 tiles to fill the chip.
__global__ __launch_bounds__(WideCfg::kThreads) void gemm_perch_wide_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = WideCfg;
    constexpr int SA = C::SA, SB = C::SB;
    __shared__ __attribute__((aligned(1024))) char lds0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[C::kStageBytes];

    Tile t;
    if (!decode_tile<C::kBN, C::kBM, false, kGroupMWide>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K, KB = p.KB;
    const int64_t wrows = p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq + t.m0 * K, clamp_bytes(t.rows * K));

    // load pieces as in the wide kernel: one chunk per lane, piece j of a
    // lane j * 64 rows below piece 0
    const int r_in = lane >> 3;
    const int chunk = 16 * ((lane & 7) ^ r_in ^ (wave & 1));
    const uint32_t go = (uint32_t)((8 * wave + r_in) * K + chunk);
    const uint32_t piece_stride = (uint32_t)(8 * C::kWaves * K);
    const int kb_in = (int)((K - chunk + kBlock - 1) / kBlock);   // kb < kb_in <=> kb * 128 + chunk < K
    auto issue = [&](char *stage, int64_t kb) __attribute__((always_inline)) {
        const uint32_t kofs = (uint32_t)kb * kBlock;
        const bool in_k = (int)kb < kb_in;
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (BI8_LDS void *)(stage + (wave + j * C::kWaves) * 1024), 16,
                in_k ? go + kofs + j * piece_stride : kOobOffset, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (BI8_LDS void *)(stage + C::kXOff + (wave + j * C::kWaves) * 1024), 16,
                in_k ? go + kofs + j * piece_stride : kOobOffset, 0, 0, 0);
    };

    const int wn = wave % C::WN, wm = wave / C::WN;
    const int rr = lane & 31, hi = lane >> 5;
    const int swz = (rr & 7) ^ ((rr >> 3) & 1);
    int frag_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) frag_off[s] = 16 * ((2 * s + hi) ^ swz);
    const int wrow0 = (wn * C::kWaveN + rr) * 128;
    const int xrow0 = C::kXOff + (wm * C::kWaveM + rr) * 128;

    i32x16 acc[SA][SB];
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0;
    auto compute = [&](const char *stage) __attribute__((always_inline)) {
        i32x4 xf[SB][4];
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xf[b][s] = *reinterpret_cast<const i32x4 *>(stage + xrow0 + b * 32 * 128 + frag_off[s]);
#pragma unroll
        for (int a = 0; a < SA; ++a) {
            i32x4 wf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wf[s] = *reinterpret_cast<const i32x4 *>(stage + wrow0 + a * 32 * 128 + frag_off[s]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int b = 0; b < SB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[s], xf[b][s], acc[a][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // block kb in lds[kb % 2]: after this wave's fills of block kb have landed
    // and every wave is past the barrier (so done with block kb - 1), block
    // kb + 1 starts filling the other stage
    issue(lds0, 0);
    int64_t kb = 0;
    for (; kb + 1 < KB; kb += 2) {
        wait_vmcnt<0>();
        lds_barrier();
        issue(lds1, kb + 1);
        compute(lds0);
        wait_vmcnt<0>();
        lds_barrier();
        issue(lds0, kb + 2);
        compute(lds1);
    }
    if (kb < KB) {   // odd block count: the last block sits in lds0
        wait_vmcnt<0>();
        lds_barrier();
        compute(lds0);
    }
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

    // Store: lane -> token column rr; element i -> weight row 8 (i / 4) + 4 hi + i % 4.
#pragma unroll
    for (int b = 0; b < SB; ++b) {
        const int64_t ml = wm * C::kWaveM + b * 32 + rr;
        if (ml >= t.rows) continue;
        const float xsv = p.xs[t.m0 + ml];
        uint16_t *yrow = p.y + (t.m0 + ml) * p.N;
#pragma unroll
        for (int a = 0; a < SA; ++a) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t n = t.n0 + wn * C::kWaveN + a * 32 + 8 * i4 + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float wsv = n + e < p.N ? t.ws[n + e] : 0.0f;
                    v[e] = (float)acc[a][b][4 * i4 + e] * (xsv * wsv);
                    if (p.bias && n + e < p.N) v[e] += bf16_bits_to_f32(p.bias[n + e]);
                }
                if (p.wide_store) {
                    if (n < p.N) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi2 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)f32_to_bf16_bits(v[e]);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Explicit instantiations: the host pass must emit a launch stub for every
// variant launched below.
template __global__ void gemm_tiled_kernel<4, 2, 2, 2, false, true, 3>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 2, 2, true, true, 3>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, true, 3>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, false, 4>(GemmArgs);
template __global__ void gemm_wide_kernel<false>(GemmArgs);
template __global__ void gemm_perch_kernel<false>(GemmArgs);
template __global__ void gemm_wide_kernel<true>(GemmArgs);

// One workgroup per 16 weight rows; 16-token tiles by M.
template <bool PC>
hipError_t launch_skinny(GemmArgs p, hipStream_t stream) {
    const int64_t tiles = (p.N + 15) / 16;
    if (tiles > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const int32_t bpw = (int32_t)((p.KB + kSkinnyWaves - 1) / kSkinnyWaves);
    const dim3 grid((unsigned)tiles), block(kSkinnyWaves * 64);
    if (p.M <= 16)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, PC>), grid, block, 0, stream, p, bpw);
    else if (p.M <= 32)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, PC>), grid, block, 0, stream, p, bpw);
    else if (p.M <= 48)
        hipLaunchKernelGGL((gemm_skinny_kernel<3, PC>), grid, block, 0, stream, p, bpw);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<4, PC>), grid, block, 0, stream, p, bpw);
    return hipGetLastError();
}

template <int WN, int WM, int SA, int SB, bool MOE, bool PING, int NS>
hipError_t launch_tiled(GemmArgs p, hipStream_t stream) {
    using C = TileCfg<WN, WM, SA, SB>;
    const int64_t total = p.tiles_m * p.tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_tiled_kernel<WN, WM, SA, SB, MOE, PING, NS>), dim3((unsigned)total), dim3(C::kThreads),
                       0, stream, p);
    return hipGetLastError();
}

template <bool MOE>
hipError_t launch_wide(GemmArgs p, hipStream_t stream) {
    const int64_t total = p.tiles_m * p.tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_wide_kernel<MOE>), dim3((unsigned)total), dim3(WideCfg::kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

GemmArgs make_args(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                   const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K) {
    GemmArgs p{};
    p.xq = xq;
    p.xs = xs;
    p.w = w;
    p.ws = ws;
    p.bias = bias;
    p.y = y;
    p.offsets = nullptr;
    p.M = M;
    p.N = N;
    p.K = K;
    p.KB = (K + kBlock - 1) / kBlock;
    p.NB = (N + kBlock - 1) / kBlock;
    p.E = 1;
    p.wide_store = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(y) & 7) == 0);
    return p;
}

}  // namespace

// Tile choice: the 256 x 256 kernel moves the fewest bytes per MAC and wins
// once its tiles fill the 256 CUs (prefill, gate_up); with fewer (down) the
// 256 x 128 kernel, with twice the tiles, is faster; 128 x 64 keeps small
// problems spread over the chip.
// The skinny kernel reads every activation row once per 16 weight rows, so
// it moves N * K * (1 + M / 16) bytes from L2 and HBM, at a rate close to
// the same for every shape; the tiled kernels read each byte far fewer times
// but, with a grid of few tiles, run one workgroup per CU at a pace per K
// block that does not depend on N.  Both times scale with K, so the choice
// is a budget on N * (16 + M), measured on each form (the per-channel tiled
// kernels have larger tiles, so fewer of them).
static bool use_skinny(int64_t M, int64_t N, bool per_channel) {
    if (M > kSkinnyMaxM) return false;
    return N * (16 + M) <= (per_channel ? kSkinnyBudgetPC : kSkinnyBudget);
}

GemmPath select_gemm_path(int64_t M, int64_t N, int64_t K) {
    (void)K;
    if (use_skinny(M, N, false)) return GemmPath::kSkinny;
    if (((M + 255) / 256) * ((N + 255) / 256) >= 256) return GemmPath::kTile256x256;
    if (((M + 127) / 128) * ((N + 255) / 256) >= 256) return GemmPath::kTile256x128;
    return GemmPath::kTile128x64;
}

// Grouped GEMM: the expert segments are ragged, so the tile count is taken
// from the mean segment length.
GemmPath select_moe_gemm_path(int64_t R, int64_t N, int64_t K, int32_t E) {
    (void)K;
    const int64_t rows_per_expert = E > 0 ? R / E : R;
    const int64_t wide_tiles = (int64_t)E * ((rows_per_expert + 255) / 256) * ((N + 255) / 256);
    return wide_tiles >= 512 ? GemmPath::kTile256x256 : GemmPath::kTile256x128;
}

hipError_t launch_gemm(GemmPath path, const int8_t *xq, const float *xs, const int8_t *w,
                       const float *ws, const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
    GemmArgs p = make_args(xq, xs, w, ws, bias, y, M, N, K);
    if (path == GemmPath::kAuto) path = select_gemm_path(M, N, K);
    switch (path) {
        case GemmPath::kSkinny: {
            if (M > kSkinnyMaxM) return hipErrorInvalidValue;
            return launch_skinny<false>(p, stream);
        }
        case GemmPath::kTile256x256:
            p.tiles_m = (M + 255) / 256;
            p.tiles_n = (N + 255) / 256;
            return launch_wide<false>(p, stream);
        case GemmPath::kTile256x128:
            p.tiles_m = (M + 127) / 128;
            p.tiles_n = (N + 255) / 256;
            return launch_tiled<4, 2, 2, 2, false, true, 3>(p, stream);
        case GemmPath::kTile128x64:
            p.tiles_m = (M + 63) / 64;
            p.tiles_n = (N + 127) / 128;
            // A grid that leaves CUs idle runs one workgroup per CU: a fourth
            // stage (96 KB of LDS) lets the loads run a block further ahead,
            // and the waves run in step (no ping-pong: with one workgroup
            // per CU its second barrier per block costs more than it hides).
            // A larger grid keeps the 72 KB ring, two workgroups per CU.
            if (p.tiles_m * p.tiles_n <= 256) return launch_tiled<4, 2, 1, 1, false, false, 4>(p, stream);
            return launch_tiled<4, 2, 1, 1, false, true, 3>(p, stream);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_per_channel(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                                   const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream) {
    GemmArgs p = make_args(xq, xs, w, ws, bias, y, M, N, K);
    p.NB = N;   // one scale per weight row
    if (use_skinny(M, N, true)) return launch_skinny<true>(p, stream);
    if (((M + 255) / 256) * ((N + 255) / 256) >= 256) {
        // enough 256 x 256 tiles to fill the chip
        p.tiles_m = (M + 255) / 256;
        p.tiles_n = (N + 255) / 256;
        const int64_t total = p.tiles_m * p.tiles_n;
        if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
        hipLaunchKernelGGL(gemm_perch_wide_kernel, dim3((unsigned)total), dim3(WideCfg::kThreads), 0, stream, p);
        return hipGetLastError();
    }
    p.tiles_m = (M + 127) / 128;
    p.tiles_n = (N + 255) / 256;
    const int64_t total = p.tiles_m * p.tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_perch_kernel<false>), dim3((unsigned)total), dim3(512), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_moe_gemm(GemmPath path, const int8_t *xq, const float *xs, const int32_t *offsets,
                           const int8_t *w, const float *ws, uint16_t *y, int64_t R, int64_t N,
                           int64_t K, int32_t E, hipStream_t stream) {
    GemmArgs p = make_args(xq, xs, w, ws, nullptr, y, R, N, K);
    p.offsets = offsets;
    p.E = E;
    if (path == GemmPath::kAuto) path = select_moe_gemm_path(R, N, K, E);
    switch (path) {
        case GemmPath::kTile256x256:
            p.tiles_m = (R + 255) / 256 + E;   // >= sum over experts of ceil(rows_e / 256)
            p.tiles_n = (N + 255) / 256;
            return launch_wide<true>(p, stream);
        case GemmPath::kTile256x128:
            p.tiles_m = (R + 127) / 128 + E;   // >= sum over experts of ceil(rows_e / 128)
            p.tiles_n = (N + 255) / 256;
            return launch_tiled<4, 2, 2, 2, true, true, 3>(p, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace bi8
