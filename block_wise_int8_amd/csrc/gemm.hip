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
    float acc_bias;           // kAccBias, kept in a scalar register (see biased_acc_to_f32)
    float *partial;           // split K: fp32 partial sums [splits, M, N] (workspace)
    int64_t kb_per_split;     // split K: K blocks per split (the last split may hold fewer)
    int8_t *aq;               // gated MoE epilogue: int8 codes [M, I] of silu(gate) * up
    float *as;                // gated MoE epilogue: their scales [M, I / 128]
    int64_t I;                // gated MoE epilogue: intermediate size (N = 2 I)
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

// 16 bytes at any byte offset `off` of a buffer whose base is 4-byte aligned:
// five aligned 4-byte loads (each range-checked on its own, so a dword past
// the buffer's end reads as zero) and byte shifts.  For rows of a K that is
// not a multiple of 16, which start at any byte.
__device__ __forceinline__ u32x4 buf_load16_any(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const uint32_t a = off & ~3u, sh = off & 3u;
    uint32_t d[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) d[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(a + 4u * i), 0, 0);
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
    return v;
}

// Keep the first n bytes of a 16-byte operand fragment (none for n <= 0, all
// for n >= 16): the part of a fragment that lies past the end of a row.
__device__ __forceinline__ i32x4 keep_bytes(i32x4 v, int64_t n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t b = n - 4 * i;
        v[i] = b >= 4 ? v[i] : (b <= 0 ? 0 : (int32_t)((uint32_t)v[i] & ((1u << (8 * b)) - 1u)));
    }
    return v;
}

// Buffer resource for bytes [p, p + n) of a tensor at any byte address: the
// base rounded down to 4 bytes (delta = p % 4 bytes before p) and the range
// rounded up to whole dwords (a dword holding a byte of the tensor lies on the
// same page, so reading all of it is safe).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_any(const int8_t *p, int64_t n, uint32_t &delta) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    delta = (uint32_t)(a & 3u);
    return make_rsrc(reinterpret_cast<const void *>(a - delta), clamp_bytes((n + delta + 3) & ~(int64_t)3));
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
// ODD: K % 16 != 0.  Rows then start at any byte: operand fragments come
// from aligned 4-byte loads (buf_load16_any), the activation bytes past K are
// zeroed (so whatever the weight fragment holds there multiplies zero), and
// blockIdx.y walks the tokens in chunks of 64, so any M runs.
template <int MT, bool PC, bool ODD>
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
    const int64_t m0 = ODD ? (int64_t)blockIdx.y * kSkinnyMaxM : 0;   // first token of this workgroup
    const int64_t mrows = p.M - m0 < kSkinnyMaxM ? p.M - m0 : kSkinnyMaxM;
    const int64_t K = p.K, KB = p.KB;

    // Each range covers only what this workgroup may read (<= 2^31 bytes since
    // K <= 2^23), so kOobOffset always lies past it.
    const int64_t wrows = p.N - n0 < 16 ? p.N - n0 : 16;
    uint32_t wd = 0, xd = 0;   // ODD: bytes between the 4-byte aligned range base and the first row
    const __amdgpu_buffer_rsrc_t wr =
        ODD ? make_rsrc_any(p.w + n0 * K, wrows * K, wd) : make_rsrc(p.w + n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr =
        ODD ? make_rsrc_any(p.xq + m0 * K, mrows * K, xd) : make_rsrc(p.xq, clamp_bytes(p.M * K));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.xs + m0 * KB, clamp_bytes(mrows * KB * 4));
    const float *ws_row = p.ws + (n0 / kBlock) * KB;
    auto load = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) __attribute__((always_inline)) {
        return as_i32x4(ODD ? buf_load16_any(r, off) : buf_load16(r, off));
    };

    const int64_t b_begin = (int64_t)wave * blocks_per_wave;
    const int64_t b_end = b_begin + blocks_per_wave < KB ? b_begin + blocks_per_wave : KB;

    // Weight loads in whole 128-byte lines (K % 16 == 0): load lane l reads
    // 16-byte chunk l % 8 of tile row l / 8 (and of row 8 + l / 8 with the
    // second load), so one load instruction covers 8 full lines.  The MFMA's A
    // operand wants lane (i, q) = (l % 16, l / 16) to hold chunk 2q + m of row
    // i for MFMA m; cross-lane permutes (ds_bpermute) move each chunk there
    // from load lane (i % 8) * 8 + 2q + m, of the first or the second load.
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int bp0 = ((lane & 7) * 8 + 2 * (lane >> 4)) * 4;   // byte index of the source lane, m = 0
    const bool upper = (lane & 15) >= 8;                        // MFMA rows 8-15: from the second load

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
            if constexpr (ODD) {
                wa[u][0] = load(wr, in0 ? (uint32_t)(wd + row * K + kk) : kOobOffset);
                wa[u][1] = load(wr, in1 ? (uint32_t)(wd + row * K + kk + 16) : kOobOffset);
            } else {   // whole lines; permuted into the MFMA layout below
                const int64_t kc = b * kBlock + lchunk * 16;
                const bool inl = ok && kc < K;
                wa[u][0] = load(wr, inl ? (uint32_t)(lrow * K + kc) : kOobOffset);
                wa[u][1] = load(wr, inl ? (uint32_t)((lrow + 8) * K + kc) : kOobOffset);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // lanes of token columns past M load nothing (zero operands)
                const int64_t tok = mt * 16 + row;   // relative to m0
                xb[u][mt][0] = i32x4{0, 0, 0, 0};
                xb[u][mt][1] = i32x4{0, 0, 0, 0};
                if constexpr (!PC) xsv[u][mt] = 0.f;
                if (tok < mrows) {
                    xb[u][mt][0] = load(xr, in0 ? (uint32_t)(xd + tok * K + kk) : kOobOffset);
                    xb[u][mt][1] = load(xr, in1 ? (uint32_t)(xd + tok * K + kk + 16) : kOobOffset);
                    if constexpr (ODD) {
                        xb[u][mt][0] = keep_bytes(xb[u][mt][0], K - kk);
                        xb[u][mt][1] = keep_bytes(xb[u][mt][1], K - kk - 16);
                    }
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
            if constexpr (!ODD) {
                i32x4 a0, a1;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int lo0 = __builtin_amdgcn_ds_bpermute(bp0, wa[u][0][d]);
                    const int hi0 = __builtin_amdgcn_ds_bpermute(bp0, wa[u][1][d]);
                    const int lo1 = __builtin_amdgcn_ds_bpermute(bp0 + 4, wa[u][0][d]);
                    const int hi1 = __builtin_amdgcn_ds_bpermute(bp0 + 4, wa[u][1][d]);
                    a0[d] = upper ? hi0 : lo0;
                    a1[d] = upper ? hi1 : lo1;
                }
                wa[u][0] = a0;
                wa[u][1] = a1;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // the block sum, accumulated onto kAccBiasBits (see biased_acc_to_f32)
                i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    wa[u][0], xb[u][mt][0], i32x4{kAccBiasBits, kAccBiasBits, kAccBiasBits, kAccBiasBits}, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[u][1], xb[u][mt][1], acc, 0, 0, 0);
                if constexpr (PC) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) yv[mt][i] += biased_acc_to_f32(acc[i], p.acc_bias);
                } else {
                    const float t = xsv[u][mt] * wsv[u];
#pragma unroll
                    for (int i = 0; i < 4; ++i) yv[mt][i] = fmaf(biased_acc_to_f32(acc[i], p.acc_bias), t, yv[mt][i]);
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
        const int64_t tok = m0 + mt * 16 + c, n = n0 + r;
        if (tok < p.M && n < p.N) {
            if constexpr (PC) s *= p.xs[tok] * p.ws[n];
            if (p.bias) s += bf16_bits_to_f32(p.bias[n]);
            p.y[tok * p.N + n] = (uint16_t)(f32x2_to_bf16x2_bits(s, 0.0f) & 0xFFFFu);
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

// Split K: target workgroups on the chip (about two per CU, each 128 x 64
// tile with a 3-stage ring taking 76 KB of LDS) and the ring depth.
#ifndef BI8_SPLITK_TARGET
#define BI8_SPLITK_TARGET 512
#endif
#ifndef BI8_SPLITK_STAGES
#define BI8_SPLITK_STAGES 3
#endif
constexpr int64_t kSplitKTarget = BI8_SPLITK_TARGET;
// The fp32 partials cost splits x M x N x 4 bytes written and read again; on
// larger outputs that traffic outweighs the shorter K runs (measured: 333 x
// 5000 x 4000 and 40 x 28672 x 4096 slower split, 64 x 8192 x 4096 and
// 129 x 1000 x 3088 20-25 % faster).
constexpr int64_t kSplitKMaxOutputs = 640 * 1024;
constexpr int kSplitKStages = BI8_SPLITK_STAGES;
constexpr int64_t kGroupMWide = 4;
// Grouped GEMM: at most this many m-tiles of one expert advance together
// along n (the workload's experts hold 4-5 tiles of 256 rows and 8-9 of 128:
// each is one group).  Measured at the MoE size: 8 and 32 within 1 %.
constexpr int64_t kGroupMMoe = 16;
#ifndef BI8_TILED_SPREAD_FILLS
#define BI8_TILED_SPREAD_FILLS 1
#endif
constexpr bool kSpreadTiled = BI8_TILED_SPREAD_FILLS;

struct Tile {
    int64_t n0;    // first weight row / output column
    int64_t m0;    // first activation row (global row of xq, xs, y)
    int64_t rows;  // valid activation rows in this tile
    const int8_t *w;
    const float *ws;
    int32_t split = -1;   // grouped tail split: this unit's split of the tile (-1: the whole tile)
    int32_t nsplit = 1;   // grouped tail split: splits of the tile
    int64_t unit = 0;     // grouped tail split: the unit's partial-sum slot
};

// Split tail of a grouped GEMM (one workgroup per CU): the tiles that exist,
// T, fill F = 256 * floor(T / 256) whole rounds of the chip's CUs; the other
// T - F run split over K into S parts each, so that their units fill one more
// round.  S = min(256 / (T - F), KB, 16), trimmed so that no split is empty;
// S = 1 when splitting would not shorten the last round.
constexpr int64_t kTailRound = 256;
constexpr int64_t kTailMaxSplitsPlan = 16;   // at most this many splits per tail tile
struct TailPlan {
    int64_t full;     // F
    int64_t tail;     // T - F
    int32_t splits;   // S
    int64_t per;      // K blocks per split
};
__device__ __forceinline__ TailPlan tail_plan(int64_t total, int64_t KB) {
    static_assert((kTailRound & (kTailRound - 1)) == 0, "power of two");
    TailPlan t;
    t.full = total & ~(kTailRound - 1);
    t.tail = total - t.full;
    // (32-bit division: tail < 256 and KB <= 2^16, K being at most 2^23)
    uint32_t s = t.tail > 0 ? (uint32_t)kTailRound / (uint32_t)t.tail : 1u;
    s = s < KB ? s : (uint32_t)KB;
    s = s < kTailMaxSplitsPlan ? s : (uint32_t)kTailMaxSplitsPlan;
    s = s < 1 ? 1 : s;
    const uint32_t kb = (uint32_t)KB;
    t.per = (kb + s - 1) / s;
    t.splits = (int32_t)((kb + (uint32_t)t.per - 1) / (uint32_t)t.per);
    return t;
}

// The tiles that exist in a grouped GEMM with BM-row tiles: sum over the
// expert segments (offsets clamped to [0, R]) of ceil(rows / BM).
template <int BM>
__device__ __forceinline__ int64_t moe_tiles_m(const GemmArgs &p) {
    int64_t n = 0;
    for (int32_t e = 0; e < p.E; ++e) {
        int64_t a = p.offsets[e], b = p.offsets[e + 1];
        a = a < 0 ? 0 : (a > p.M ? p.M : a);
        b = b < a ? a : (b > p.M ? p.M : b);
        n += (b - a + BM - 1) / BM;
    }
    return n;
}

// Tile `tid` of the grouped order over tiles_m m-tiles: groups of GM m-tiles
// advance together along n, so the tiles that share a weight tile run side by
// side.  For the grouped GEMM the groups follow the expert segments: expert e's
// m-tiles (found by walking the segments) in groups of at most kGroupMMoe, so
// that no group mixes two experts' weights (groups across segment boundaries
// read both experts' weight tiles, and most of the weights twice).
template <int BN, int BM, bool MOE, int64_t GM>
__device__ __forceinline__ bool tile_at(const GemmArgs &p, int64_t tid, int64_t tiles_m, Tile &t) {
    // (32-bit division: tid < 2^31 and GM * tiles_n < 2^31, both launch limits)
    if constexpr (!MOE) {
        const uint32_t span = (uint32_t)(GM * p.tiles_n);
        const uint32_t group = (uint32_t)tid / span;
        const int64_t first_m = (int64_t)group * GM;
        const uint32_t gsize = (uint32_t)(tiles_m - first_m < GM ? tiles_m - first_m : GM);
        const uint32_t in = (uint32_t)tid - group * span;
        t.n0 = (int64_t)(in / gsize) * BN;
        t.m0 = (first_m + in % gsize) * BM;
        t.rows = p.M - t.m0 < BM ? p.M - t.m0 : BM;
        t.w = p.w;
        t.ws = p.ws;
        return true;
    } else {
        int64_t rem = tid;
        for (int32_t e = 0; e < p.E; ++e) {
            // clamp to [0, R] so that offsets breaking the precondition can
            // never address rows outside xq / y
            int64_t a = p.offsets[e], b = p.offsets[e + 1];
            a = a < 0 ? 0 : (a > p.M ? p.M : a);
            b = b < a ? a : (b > p.M ? p.M : b);
            const int64_t cnt = (b - a + BM - 1) / BM;
            const int64_t espan = cnt * p.tiles_n;
            if (rem < espan) {
                const uint32_t span = (uint32_t)(kGroupMMoe * p.tiles_n);
                const uint32_t group = (uint32_t)rem / span;
                const int64_t first_m = (int64_t)group * kGroupMMoe;
                const uint32_t gsize = (uint32_t)(cnt - first_m < kGroupMMoe ? cnt - first_m : kGroupMMoe);
                const uint32_t in = (uint32_t)rem - group * span;
                t.n0 = (int64_t)(in / gsize) * BN;
                t.m0 = a + (first_m + in % gsize) * BM;
                t.rows = b - t.m0 < BM ? b - t.m0 : BM;
                t.w = p.w + (int64_t)e * p.N * p.K;
                t.ws = p.ws + (int64_t)e * p.NB * p.KB;
                return true;
            }
            rem -= espan;
        }
        return false;
    }
}

template <int BN, int BM, bool MOE, int64_t GM = kGroupM, bool TAIL = false>
__device__ __forceinline__ bool decode_tile(const GemmArgs &p, Tile &t) {
    // MoE: the grid holds an upper bound of m-tiles (the segments' lengths are
    // only known on the device); the tiles that exist are counted here and
    // spread evenly over the XCDs, and the surplus workgroups exit.  (Mapped
    // over the whole grid instead, the missing tiles -- all at the end of the
    // order -- left the last XCD nearly idle: at R = 8192 over 8 experts the
    // w13 grid gave six XCDs 560 tiles each and one XCD 56.)
    // TAIL: workgroups [0, F) take the whole tiles of the full rounds (spread
    // over the XCDs as above), workgroup F + u split unit u of the tail: tile
    // F + u / S, split u % S.
    static_assert(!TAIL || MOE, "split tails are the grouped GEMM's");
    int64_t tiles_m = p.tiles_m;
    if constexpr (MOE) tiles_m = moe_tiles_m<BM>(p);
    const int64_t total = tiles_m * p.tiles_n;
    int64_t tid;
    if constexpr (MOE) {
        int64_t balanced = total;
        if constexpr (TAIL) {
            const TailPlan tp = tail_plan(total, p.KB);
            if (tp.splits > 1) {
                balanced = tp.full;
                if ((int64_t)blockIdx.x >= tp.full) {
                    const int64_t u = (int64_t)blockIdx.x - tp.full;
                    if (u >= tp.tail * tp.splits) return false;
                    tid = tp.full + u / tp.splits;
                    t.split = (int32_t)(u % tp.splits);
                    t.nsplit = tp.splits;
                    t.unit = u;
                    balanced = -1;
                }
            }
        }
        if (balanced >= 0) {
            const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
            const int64_t q = balanced >> 3, r = balanced & 7;
            if (slot >= q + (xcd < r ? 1 : 0)) return false;
            tid = xcd * q + (xcd < r ? xcd : r) + slot;
        }
    } else {
        tid = xcd_remap(blockIdx.x, total);
    }
    return tile_at<BN, BM, MOE, GM>(p, tid, tiles_m, t);
}

// PING: the two wave groups (rows wm = 0 and wm = 1 of the wave grid; waves w
// and w + 4 share a SIMD) run half a K step apart.  Per K step there are two
// barriers; between them one group issues its MFMAs while the other converts
// and rescales its previous block (VALU), so each SIMD keeps its matrix core
// and its vector ALU busy at the same time.
// SPLIT: split K.  Workgroup (tile, blockIdx.y) sums only the K blocks
// [blockIdx.y * kb_per_split, + kb_per_split) and stores its fp32 partial sums
// (no bias, no rounding) in p.partial[blockIdx.y]; splitk_reduce_kernel adds
// the splits up.  The ring and the scale batches count blocks from the first
// one of the split.
template <int WN, int WM, int SA, int SB, bool MOE, bool PING, int NS, bool SPLIT>
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
    // grouped with SPLIT: the full rounds' tiles whole, the tail's split over K
    if (!decode_tile<C::kBN, C::kBM, MOE, kGroupM, MOE && SPLIT>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K;
    // K blocks of this workgroup: [kb0, kb0 + KB); chunks at or past kend read
    // zero.  Dense split K: split blockIdx.y of kb_per_split blocks; grouped
    // tail: split t.split of the tail plan's `per` blocks.
    int64_t kb0 = 0, KB = p.KB;
    if constexpr (SPLIT && !MOE) {
        kb0 = (int64_t)blockIdx.y * p.kb_per_split;
        KB = p.KB - kb0 < p.kb_per_split ? p.KB - kb0 : p.kb_per_split;
    }
    if constexpr (SPLIT && MOE) {
        if (t.split >= 0) {
            const int64_t per = (p.KB + t.nsplit - 1) / t.nsplit;
            kb0 = (int64_t)t.split * per;
            KB = p.KB - kb0 < per ? p.KB - kb0 : per;
        }
    }
    const int64_t kend = SPLIT ? ((kb0 + KB) * kBlock < K ? (kb0 + KB) * kBlock : K) : K;

    // Each range covers only this tile's rows (<= 2^31 bytes since K <= 2^23),
    // so kOobOffset always lies past it.
    const int64_t wrows = p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.xq + t.m0 * K, clamp_bytes(t.rows * K));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.xs + t.m0 * p.KB, clamp_bytes(t.rows * p.KB * 4));

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
    // (lb: the block's index within this workgroup's run; kb0 + lb: in K)
    // part: -1 every load of the stage; 0 / 1 the scales and the first half
    // of the pieces / the second half (ping-pong spreads a stage's loads over
    // the two halves of a step)
    auto issue = [&](char *stage, int64_t lb, const int part = -1) __attribute__((always_inline)) {
        const int64_t k0 = (kb0 + lb) * kBlock;
        const uint32_t kofs = (uint32_t)k0;
        auto mine = [&](int j, int n) { return part < 0 || (part == 0) == (j < (n + 1) / 2); };
        if (part <= 0 && (lb & (C::kSB - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < C::kScaleLoads; ++j) {
                const int f = (wave * C::kScaleLoads + j) * 64 + lane;
                const int64_t g = lb + (f & (C::kSB - 1));
                sv[j] = buf_load_f32(sr, g < KB ? (uint32_t)(((f / C::kSB) * p.KB + kb0 + g) * 4) : kOobOffset);
            }
        }
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            if (mine(j, C::kWLoads))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (BI8_LDS void *)(stage + C::kWOff + (wave + j * C::kWaves) * 1024), 16,
                    (k0 + wchunk[j] < kend) ? wgo[j] + kofs : kOobOffset, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            if (mine(j, C::kXLoads))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (BI8_LDS void *)(stage + C::kXOff + (wave + j * C::kWaves) * 1024), 16,
                    (k0 + xchunk[j] < kend) ? xgo[j] + kofs : kOobOffset, 0, 0, 0);
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
    // The wave's weight-scale row (from this workgroup's first block), read
    // through the constant address space so that the wave-uniform loads
    // become scalar loads (the scales are never written while the kernel runs).
    const BI8_CONST float *ws_row = reinterpret_cast<const BI8_CONST float *>(
        reinterpret_cast<uintptr_t>(t.ws + nbw * p.KB + kb0));

    // each block sum starts from kAccBiasBits (see biased_acc_to_f32)
    i32x16 bias16;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias16[i] = kAccBiasBits;
    f32x16 y[SA][SB];
#pragma unroll
    for (int a = 0; a < SA; ++a)
#pragma unroll
        for (int b = 0; b < SB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) y[a][b][i] = 0.f;

    // MFMA phase: the block's int32 sums for the wave's sub-tiles, plus the
    // scales the rescale will need (read now: the stage may be refilled before
    // the rescale runs).  Two buffers (buf): without ping-pong, the rescale of
    // block kb - 1 runs while block kb's MFMAs execute, so it is off the
    // per-block chain of barrier, fragment reads and MFMAs (with ping-pong
    // only buffer 0 is used).
    i32x16 acc[2][SA][SB];
    float xsv[2][SB], wsv[2] = {0.f, 0.f};
    auto mma = [&](const char *stage, int64_t kb, const int buf) __attribute__((always_inline)) {
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
            xsv[buf][b] = xsl[(kb / C::kSB) & 1][srow[b] + (kb & (C::kSB - 1))];
        wsv[buf] = ws_row[kb];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < SA; ++a)
#pragma unroll
                for (int b = 0; b < SB; ++b)
                    acc[buf][a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        wf[a][s], xf[b][s], s == 0 ? bias16 : acc[buf][a][b], 0, 0, 0);
        // the MFMAs belong to this phase
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < SB; ++b) asm volatile("" : "+v"(acc[buf][a][b]));
    };
    // Rescale phase: y += float(acc) * (xs * ws) per sub-tile.
    auto epi = [&](const int buf) __attribute__((always_inline)) {
        float tb[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) tb[b] = xsv[buf][b] * wsv[buf];
#pragma unroll
        for (int a = 0; a < SA; ++a)
#pragma unroll
            for (int b = 0; b < SB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    y[a][b][i] = fmaf(biased_acc_to_f32(acc[buf][a][b][i], p.acc_bias), tb[b], y[a][b][i]);
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
    // kb are complete.  Without ping-pong, block kb's sums use buffer kb % 2:
    // the ring depth is even, so that is the unrolled step's index % 2.
    static_assert(PING || NS % 2 == 0, "the two accumulator buffers alternate with the ring's steps");
    auto step = [&](const int group, char *cur, char *ahead, int64_t kb, const int buf)
                    __attribute__((always_inline)) {
        wait_stage(kb);
        lds_barrier();
        issue(ahead, kb + NS - 1, kSpreadTiled && PING ? 0 : -1);
        if (!PING) {
            mma(cur, kb, buf);
            if (kb > 0) epi(buf ^ 1);   // block kb - 1, under block kb's MFMAs
        } else if (group == 0) {
            mma(cur, kb, 0);
            lds_barrier();
            if (kSpreadTiled) issue(ahead, kb + NS - 1, 1);
            epi(0);
        } else {
            if (kb > 0) epi(0);   // block kb - 1
            lds_barrier();
            if (kSpreadTiled) issue(ahead, kb + NS - 1, 1);
            mma(cur, kb, 0);
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
            for (int i = 0; i < NS; ++i) step(group, lds(i), lds((i + NS - 1) % NS), kb + i, i & 1);
        }
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (kb < KB) step(group, lds(i), lds((i + NS - 1) % NS), kb++, i & 1);
        if (PING && group == 1) epi(0);   // the last block
        if (!PING) {                      // the last block, in buffer (KB - 1) % 2
            if ((KB - 1) & 1)
                epi(1);
            else
                epi(0);
        }
    };
    if (!PING || wm == 0)
        run(0);
    else
        run(1);
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

    // Store.  32x32 result layout: lane -> token column (lane & 31); element i
    // -> weight row 8 * (i / 4) + 4 * (lane >> 5) + (i % 4).
    if constexpr (SPLIT && MOE) {
        if (t.split >= 0) {
            // the unit's fp32 partial sums in its slot, [BM tile rows][BN tile
            // columns], every row and column (moe_tail_reduce_kernel reads
            // only the valid ones)
            float *slot = p.partial + t.unit * (int64_t)(C::kBM * C::kBN);
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                float *prow = slot + (int64_t)(wm * C::kWaveM + b * 32 + rr) * C::kBN;
#pragma unroll
                for (int a = 0; a < SA; ++a)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const int c = wn * C::kWaveN + a * 32 + 8 * i4 + 4 * hi;
                        *reinterpret_cast<f32x4 *>(prow + c) =
                            f32x4{y[a][b][4 * i4], y[a][b][4 * i4 + 1], y[a][b][4 * i4 + 2], y[a][b][4 * i4 + 3]};
                    }
            }
            return;
        }
    } else if constexpr (SPLIT) {
        // fp32 partial sums of this split, no bias, no rounding
        float *part = p.partial + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int64_t ml = wm * C::kWaveM + b * 32 + rr;
            if (ml >= t.rows) continue;
            float *prow = part + (t.m0 + ml) * p.N;
#pragma unroll
            for (int a = 0; a < SA; ++a) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int64_t n = t.n0 + wn * C::kWaveN + a * 32 + 8 * i4 + 4 * hi;
                    if (p.wide_store) {
                        if (n < p.N)
                            *reinterpret_cast<f32x4 *>(prow + n) =
                                f32x4{y[a][b][4 * i4], y[a][b][4 * i4 + 1], y[a][b][4 * i4 + 2], y[a][b][4 * i4 + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N) prow[n + e] = y[a][b][4 * i4 + e];
                    }
                }
            }
        }
        return;
    }
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
                        const uint32_t lo = f32x2_to_bf16x2_bits(v[0], v[1]);
                        const uint32_t hi2 = f32x2_to_bf16x2_bits(v[2], v[3]);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)(f32x2_to_bf16x2_bits(v[e], 0.0f) & 0xFFFFu);
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
//
// SILU (grouped form only): the w13 projection with the SiLU gating and the
// requantisation of its output in the epilogue.  A workgroup owns 128 columns
// [i0, i0 + 128) of the intermediate activation: weight rows i0.. of the gate
// half fill tile rows 0-127 (waves wn = 0) and rows I + i0.. of the up half
// tile rows 128-255 (waves wn = 1), so a gate wave and the up wave of the
// same wm hold gate and up of the same (token, column) in the same lane and
// register.  The epilogue rounds both to bf16 (the value the unfused
// projection stores), passes up through LDS, and the gate waves form
// bf16(silu(g) * u), the 128-group scale of each token (the group lies in
// lanes l and l ^ 32) and its int8 codes -- the same operations in the same
// precision as silu_mul_quant_kernel, so the result is bit-identical to the
// projection followed by that kernel.  Requires I % 128 == 0.
#ifndef BI8_WIDE_SPREAD_FILLS
#define BI8_WIDE_SPREAD_FILLS 1
#endif
constexpr bool kSpreadFills = BI8_WIDE_SPREAD_FILLS;
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

template <bool MOE, bool SILU>
__global__ __launch_bounds__(WideCfg::kThreads) void gemm_wide_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = WideCfg;
    constexpr int SA = C::SA, SB = C::SB;
    __shared__ __attribute__((aligned(1024))) char lds0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[C::kStageBytes];
    __shared__ float xsl[2][C::kBM * C::kSB];

    static_assert(!SILU || MOE, "the gated epilogue is the grouped w13 projection's");
    Tile t;
    // SILU: t.n0 = i0, the first of the workgroup's 128 intermediate columns
    if (!decode_tile<SILU ? C::kBN / 2 : C::kBN, C::kBM, MOE, kGroupMWide>(p, t)) return;
    if (t.rows <= 0) return;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t K = p.K, KB = p.KB;

    // SILU: the load pieces j = 0, 1 (tile rows 0-127) read gate rows i0..
    // through wr, the pieces j = 2, 3 (tile rows 128-255) up rows I + i0..
    // through wr_up, at the offsets of pieces j - 2.
    const int64_t wrows = SILU ? C::kBN / 2 : (p.N - t.n0 < C::kBN ? p.N - t.n0 : C::kBN);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(t.w + t.n0 * K, clamp_bytes(wrows * K));
    const __amdgpu_buffer_rsrc_t wr_up = SILU ? make_rsrc(t.w + (p.I + t.n0) * K, clamp_bytes(wrows * K)) : wr;
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

    // The loads of block kb named by `mask`: bit j weight piece j, bit 4 + j
    // activation piece j, bit 8 the scale batch (when kb starts one).  A
    // block's fills are spread over its sub-tiles instead of queueing in the
    // address unit all at once.
    auto issue = [&](char *stage, int64_t kb, unsigned mask) __attribute__((always_inline)) {
        const uint32_t kofs = (uint32_t)kb * kBlock;
        if ((mask & 0x100u) && (kb & (C::kSB - 1)) == 0) {
            // The batch of activation scales goes straight to LDS, 4 bytes a
            // lane.  Entries past the last K block read the next row's scales
            // (or zero past the end of xs): they are never used, so no check.
#pragma unroll
            for (int j = 0; j < C::kScaleLoads; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    sr, (BI8_LDS void *)&xsl[(kb / C::kSB) & 1][(wave * C::kScaleLoads + j) * 64], 4,
                    sofs[j] + (uint32_t)kb * 4u, 0, 0, 0);
        }
        // Only the activation chunks past K are zeroed: the weight bytes there
        // (the next row's, or zero past the buffer) multiply zeros.
        const bool in_k = (int)kb < kb_in;
#pragma unroll
        for (int j = 0; j < C::kWLoads; ++j)
            if (mask & (1u << j))
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    SILU && j >= C::kWLoads / 2 ? wr_up : wr,
                    (BI8_LDS void *)(stage + (wave + j * C::kWaves) * 1024), 16,
                    go + kofs + (SILU && j >= C::kWLoads / 2 ? j - C::kWLoads / 2 : j) * piece_stride, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C::kXLoads; ++j)
            if (mask & (1u << (4 + j)))
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
    // Sub-tile row block b of wave wm holds tile rows b * 128 + wm * 32 + [0, 32):
    // a tile of at most 128 rows (the last of an expert's segment, say) keeps
    // every wave's rows in b = 0, and a wave whose row blocks lie past the
    // tile's rows skips their MFMAs, fragment reads and rescales (ACT below).
    auto trow = [&](int b) { return b * (C::kBM / SB) + wm * 32 + rr; };
    const int xrow0 = C::kXOff + (wm * 32 + rr) * 128;
    int srow[SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) srow[b] = trow(b) * C::kSB;
    // row blocks of this wave holding a row of the tile (a block past the
    // rows implies every later one is)
    int act = 0;
#pragma unroll
    for (int b = 0; b < SB; ++b) act += b * (C::kBM / SB) + wm * 32 < t.rows;
    act = __builtin_amdgcn_readfirstlane(act);

    int64_t nbw = (SILU ? t.n0 + wn * p.I : t.n0 + wn * C::kWaveN) / kBlock;
    if (nbw > p.NB - 1) nbw = p.NB - 1;
    const BI8_CONST float *ws_row = reinterpret_cast<const BI8_CONST float *>(
        reinterpret_cast<uintptr_t>(t.ws + nbw * KB));
    // The weight scale of a block is a scalar load issued one block ahead:
    // scalar loads complete out of order, so a use right after the load would
    // wait for every outstanding LDS read as well.
    float ws_cur = ws_row[0];

    // (the block sums start from zero here: a bias constant would take 16 of
    // the registers the 8 sub-tiles' accumulators already fill)
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
    // ACT: the wave's active row blocks (b < ACT)
    auto read_first = [&](auto actc, const char *stage, int64_t kb) __attribute__((always_inline)) {
        constexpr int ACT = decltype(actc)::value;
#pragma unroll
        for (int b = 0; b < ACT; ++b) xsv[b] = xsl[(kb / C::kSB) & 1][srow[b] + (kb & (C::kSB - 1))];
        if constexpr (ACT > 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s) wf0[s] = *reinterpret_cast<const i32x4 *>(stage + wrow0 + frag_off[s]);
        }
#pragma unroll
        for (int b = 0; b < ACT; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xf[b][s] = *reinterpret_cast<const i32x4 *>(stage + xrow0 + b * (C::kBM / SB) * 128 + frag_off[s]);
        wsv = ws_cur;
        ws_cur = ws_row[kb + 1 < KB ? kb + 1 : KB - 1];   // next block's, issued a block ahead
    };
    // Block kb + 1 is in LDS once this wave's fills have landed and every wave
    // is past the barrier (which also ends every read of block kb): read its
    // first fragments from `nxt`.  After the last block this reads stale LDS
    // that nothing uses.
    auto advance = [&](auto actc, const char *nxt, int64_t kb) __attribute__((always_inline)) {
        wait_vmcnt<0>();
        lds_barrier();
        read_first(actc, nxt, kb + 1);
    };

    // One K block: first the fills of block kb + 1 into the other stage (its
    // previous block was finished before the last barrier; past the last
    // block they read zeros), then the sub-tiles in the order (a, b) = (0,0),
    // (0,1), (1,0), ...; the rescale of each sub-tile is issued after the next
    // sub-tile's MFMAs, and the last one after the next block's first
    // fragment reads.
    auto compute = [&](auto actc, const char *stage, char *nxt, int64_t kb) __attribute__((always_inline)) {
        constexpr int ACT = decltype(actc)::value;
        // past the last block nothing is loaded (the stage it would fill is
        // never read)
        const bool more = kb + 1 < KB;
        if ((!kSpreadFills || ACT == 0) && more) issue(nxt, kb + 1, 0x1FFu);
        if constexpr (ACT == 0) {
            advance(actc, nxt, kb);
            return;
        }
        float tb[SB];
#pragma unroll
        for (int b = 0; b < ACT; ++b) tb[b] = xsv[b] * wsv;
        i32x16 acc[2];
#pragma unroll
        for (int a = 0; a < SA; ++a) {
            i32x4 wf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wf[s] = a == 0 ? wf0[s]
                               : *reinterpret_cast<const i32x4 *>(stage + wrow0 + a * 32 * 128 + frag_off[s]);
#pragma unroll
            for (int b = 0; b < ACT; ++b) {
                const int j = a * ACT + b;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[j & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[s], xf[b][s],
                                                                         s == 0 ? zero16 : acc[j & 1], 0, 0, 0);
                // weight and activation piece j after sub-tile j's MFMAs (j < 4;
                // spread over all eight sub-tiles the last fills came late)
                if (kSpreadFills && j < 4 && more) issue(nxt, kb + 1, (0x11u << j) | (j == 0 ? 0x100u : 0u));
                if (j > 0) {
                    const int pa = (j - 1) / ACT, pb = (j - 1) % ACT;
                    rescale(acc[(j - 1) & 1], y[pa][pb], tb[pb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last sub-tile's MFMAs stay ahead of the barrier as well
        asm volatile("" ::"v"(acc[(SA * ACT - 1) & 1]));
        advance(actc, nxt, kb);
        rescale(acc[(SA * ACT - 1) & 1], y[SA - 1][ACT - 1], tb[ACT - 1]);
    };

    auto run = [&](auto actc) __attribute__((always_inline)) {
        issue(lds0, 0, 0x1FFu);
        wait_vmcnt<0>();
        lds_barrier();
        read_first(actc, lds0, 0);
        for (int64_t kb = 0;; kb += 2) {
            // block kb in lds0, block kb + 1 in lds1
            compute(actc, lds0, lds1, kb);
            if (kb + 1 >= KB) break;
            compute(actc, lds1, lds0, kb + 1);
            if (kb + 2 >= KB) break;
        }
    };
    // (a wave with no row of the tile takes the one-block variant: its
    // block reads zeros).  Only the gated kernel takes two variants: in the
    // others the allocation of the pair spills in the full variant's loop,
    // and the reload waits behind the outstanding fills.
    static_assert(SB == 2, "row-block variants");
    if constexpr (SILU) {
        if (act == SB)
            run(std::integral_constant<int, SB>{});
        else
            run(std::integral_constant<int, 1>{});
    } else {
        run(std::integral_constant<int, SB>{});
    }
    wait_vmcnt<0>();   // no LDS fill may outlive the workgroup

    if constexpr (SILU) {
        // Gate wave (wn = 0) and up wave (wn = 1) of one wm share the work:
        // the gate wave finishes columns a = 0, 1 of its sub-tiles, the up wave
        // a = 2, 3 (each needs the other's value there), so all four SIMDs
        // take part.  Values travel as bf16 through LDS: (a, b, register i) of
        // lane l at slot(b, a) + (i / 8) KB + 16 l + 2 (i % 8).  The group
        // maximum of a token's 128 columns is then combined over lanes l and
        // l ^ 32 of both waves.
        __syncthreads();   // every wave is past its last fragment read: the stages are free
        char *xbuf = lds0;
        float *mbuf = &xsl[0][0];   // [wm][wn][b][32] partial group maxima
        auto slot = [&](int b, int a) { return xbuf + ((wm * SB + b) * SA + a) * 2048 + lane * 16; };
        auto give = [&](auto a0c) __attribute__((always_inline)) {
            constexpr int A0 = decltype(a0c)::value;
#pragma unroll
            for (int b = 0; b < SB; ++b)
#pragma unroll
                for (int a = A0; a < A0 + 2; ++a)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        u32x4 v;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            v[j] = f32x2_to_bf16x2_bits(y[a][b][8 * h + 2 * j], y[a][b][8 * h + 2 * j + 1]);
                        *reinterpret_cast<u32x4 *>(slot(b, a) + h * 1024) = v;
                    }
        };
        if (wn == 0)
            give(std::integral_constant<int, 2>{});
        else
            give(std::integral_constant<int, 0>{});
        __syncthreads();

        // a = bf16(silu(g) * u) over the wave's own columns, in place of y;
        // the per-element SiLU takes its far-negative branch only in a wave
        // that holds such a gate value (silu_times with g >= -80 is the plain
        // expression)
        float amax[SB];
        auto gate_up = [&](auto a0c, auto gatec) __attribute__((always_inline)) {
            constexpr int A0 = decltype(a0c)::value;
            constexpr bool GATE = decltype(gatec)::value;
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                float gv[32], uv[32];
                float gmin = 0.0f;
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const u32x4 pv = *reinterpret_cast<const u32x4 *>(slot(b, A0 + aa) + h * 1024);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int i = 8 * h + 2 * j, k = 16 * aa + i;
                            const uint32_t ob = f32x2_to_bf16x2_bits(y[A0 + aa][b][i], y[A0 + aa][b][i + 1]);
                            const float o0 = bf16_bits_to_f32(ob & 0xFFFFu), o1 = bf16_bits_to_f32(ob >> 16);
                            const float p0 = bf16_bits_to_f32(pv[j] & 0xFFFFu), p1 = bf16_bits_to_f32(pv[j] >> 16);
                            gv[k] = GATE ? o0 : p0;
                            gv[k + 1] = GATE ? o1 : p1;
                            uv[k] = GATE ? p0 : o0;
                            uv[k + 1] = GATE ? p1 : o1;
                            gmin = fminf(gmin, fminf(gv[k], gv[k + 1]));
                        }
                    }
                float am = 0.0f;
                const bool far = __any(gmin < -80.0f);
#pragma unroll
                for (int k = 0; k < 32; k += 2) {
                    float s0, s1;
                    if (far) {
                        s0 = silu_times(gv[k], uv[k]);
                        s1 = silu_times(gv[k + 1], uv[k + 1]);
                    } else {
                        s0 = gv[k] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gv[k] * -1.44269504f)) * uv[k];
                        s1 = gv[k + 1] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gv[k + 1] * -1.44269504f)) *
                             uv[k + 1];
                    }
                    const uint32_t ab = f32x2_to_bf16x2_bits(s0, s1);
                    const float a0 = bf16_bits_to_f32(ab & 0xFFFFu), a1 = bf16_bits_to_f32(ab >> 16);
                    y[A0 + k / 16][b][k % 16] = a0;
                    y[A0 + k / 16][b][k % 16 + 1] = a1;
                    am = fmaxf(am, fmaxf(fabsf(a0), fabsf(a1)));
                }
                am = fmaxf(am, __shfl_xor(am, 32));
                amax[b] = am;
                if (hi == 0) mbuf[((wm * 2 + wn) * SB + b) * 32 + rr] = am;
            }
        };
        if (wn == 0)
            gate_up(std::integral_constant<int, 0>{}, std::true_type{});
        else
            gate_up(std::integral_constant<int, 2>{}, std::false_type{});
        __syncthreads();

        // codes of the wave's own columns and (gate wave) the group scale;
        // quant_code's division fallback runs only in a wave that needs it
        const int64_t I = p.I, IB = I / kBlock, g = t.n0 / kBlock;
        auto quant_store = [&](auto a0c) __attribute__((always_inline)) {
            constexpr int A0 = decltype(a0c)::value;
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const float am = fmaxf(amax[b], mbuf[((wm * 2 + (wn ^ 1)) * SB + b) * 32 + rr]);
                const float sc = am / 127.0f;
                const float rs = __builtin_amdgcn_rcpf(sc);
                uint32_t code[2][4];
                float dmax = 0.0f;
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        uint32_t c = 0u;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = y[A0 + aa][b][4 * i4 + e] * rs;
                            float q = rintf(v);
                            dmax = fmaxf(dmax, fabsf(v - q));
                            q = fminf(fmaxf(q, -127.0f), 127.0f);
                            c |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * e);
                        }
                        code[aa][i4] = c;
                    }
                // the products are finite whenever am and rs are; otherwise, or
                // near a half-integer, take quant_code itself
                const bool fine = dmax < 0.5f - 0x1p-14f && rs * 0.0f == 0.0f && am * 0.0f == 0.0f;
                if (__any(sc != 0.0f && !fine)) {
#pragma unroll
                    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            uint32_t c = 0u;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                c |= ((uint32_t)quant_code(y[A0 + aa][b][4 * i4 + e], sc, rs) & 0xFFu) << (8 * e);
                            code[aa][i4] = c;
                        }
                }
                const int64_t ml = trow(b);
                if (ml >= t.rows) continue;
                const int64_t r = t.m0 + ml;
                int8_t *arow = p.aq + r * I + t.n0;
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)
                        *reinterpret_cast<uint32_t *>(arow + (A0 + aa) * 32 + 8 * i4 + 4 * hi) =
                            sc != 0.0f ? code[aa][i4] : 0u;
                if (A0 == 0 && hi == 0) p.as[r * IB + g] = sc;
            }
        };
        if (wn == 0)
            quant_store(std::integral_constant<int, 0>{});
        else
            quant_store(std::integral_constant<int, 2>{});
        return;
    }

#pragma unroll
    for (int b = 0; b < SB; ++b) {
        const int64_t ml = trow(b);
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
                        const uint32_t lo = f32x2_to_bf16x2_bits(v[0], v[1]);
                        const uint32_t hi2 = f32x2_to_bf16x2_bits(v[2], v[3]);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)(f32x2_to_bf16x2_bits(v[e], 0.0f) & 0xFFFFu);
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
                        const uint32_t lo = f32x2_to_bf16x2_bits(v[0], v[1]);
                        const uint32_t hi2 = f32x2_to_bf16x2_bits(v[2], v[3]);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)(f32x2_to_bf16x2_bits(v[e], 0.0f) & 0xFFFFu);
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
                        const uint32_t lo = f32x2_to_bf16x2_bits(v[0], v[1]);
                        const uint32_t hi2 = f32x2_to_bf16x2_bits(v[2], v[3]);
                        *reinterpret_cast<uint2 *>(yrow + n) = make_uint2(lo, hi2);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N) yrow[n + e] = (uint16_t)(f32x2_to_bf16x2_bits(v[e], 0.0f) & 0xFFFFu);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Explicit instantiations: the host pass must emit a launch stub for every
// variant launched below.
template __global__ void gemm_tiled_kernel<4, 2, 2, 2, false, true, 3, false>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 2, 2, true, true, 3, false>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, true, 3, false>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, false, 4, false>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, true, 3, true>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 1, 1, false, false, 4, true>(GemmArgs);
template __global__ void gemm_tiled_kernel<4, 2, 2, 2, true, true, 3, true>(GemmArgs);
template __global__ void gemm_wide_kernel<false, false>(GemmArgs);
template __global__ void gemm_perch_kernel<false>(GemmArgs);
template __global__ void gemm_wide_kernel<true, false>(GemmArgs);
template __global__ void gemm_wide_kernel<true, true>(GemmArgs);

// One workgroup per 16 weight rows; 16-token tiles by M.  ODD (K % 16 != 0):
// the same for every M, in chunks of 64 tokens along the grid's y.
template <bool PC, bool ODD>
hipError_t launch_skinny(GemmArgs p, hipStream_t stream) {
    const int64_t tiles = (p.N + 15) / 16;
    const int64_t chunks = ODD ? (p.M + kSkinnyMaxM - 1) / kSkinnyMaxM : 1;
    if (tiles > 0x7FFFFFFFll || chunks > 65535) return hipErrorInvalidValue;
    if (tiles == 0 || chunks == 0) return hipSuccess;
    const int32_t bpw = (int32_t)((p.KB + kSkinnyWaves - 1) / kSkinnyWaves);
    const dim3 grid((unsigned)tiles, (unsigned)chunks), block(kSkinnyWaves * 64);
    if (p.M <= 16)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, PC, ODD>), grid, block, 0, stream, p, bpw);
    else if (p.M <= 32)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, PC, ODD>), grid, block, 0, stream, p, bpw);
    else if (p.M <= 48)
        hipLaunchKernelGGL((gemm_skinny_kernel<3, PC, ODD>), grid, block, 0, stream, p, bpw);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<4, PC, ODD>), grid, block, 0, stream, p, bpw);
    return hipGetLastError();
}

template <int WN, int WM, int SA, int SB, bool MOE, bool PING, int NS, bool SPLIT = false>
hipError_t launch_tiled(GemmArgs p, hipStream_t stream, int32_t splits = 1) {
    using C = TileCfg<WN, WM, SA, SB>;
    const int64_t total = p.tiles_m * p.tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7FFFFFFFll || splits < 1 || splits > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_tiled_kernel<WN, WM, SA, SB, MOE, PING, NS, SPLIT>),
                       dim3((unsigned)total, (unsigned)splits), dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

// y[m, n] = bf16(sum over the splits, in split order, of partial[z, m, n]
// (+ bias[n])); four outputs of one row per thread when N % 4 == 0.
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partial, int32_t splits,
                                                            int64_t M, int64_t N, const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ y) {
    const int64_t MN = M * N;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (VEC ? 4 : 1);
    if (i >= MN) return;
    if constexpr (VEC) {
        f32x4 acc = *reinterpret_cast<const f32x4 *>(partial + i);
        for (int32_t z = 1; z < splits; ++z) acc += *reinterpret_cast<const f32x4 *>(partial + z * MN + i);
        if (bias) {
            const int64_t n = i % N;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += bf16_bits_to_f32(bias[n + e]);
        }
        *reinterpret_cast<uint2 *>(y + i) =
            make_uint2(f32x2_to_bf16x2_bits(acc[0], acc[1]), f32x2_to_bf16x2_bits(acc[2], acc[3]));
    } else {
        float acc = partial[i];
        for (int32_t z = 1; z < splits; ++z) acc += partial[z * MN + i];
        if (bias) acc += bf16_bits_to_f32(bias[i % N]);
        y[i] = (uint16_t)(f32x2_to_bf16x2_bits(acc, 0.0f) & 0xFFFFu);
    }
}

// Split tail of the grouped GEMM (BN x BM tiles): for each row r of each tail
// tile F + i, the S partial sums of its units added in split order and stored
// as bf16 -- the plan recomputed exactly as the GEMM's decoder computed it.
// A fixed grid (the tail's size is only known on the device); its waves take
// the (tile, row) pairs in turn, lane l columns
// [4l, 4l + 4) of every 256 columns, every split's load issued before the
// first add.
constexpr int kTailMaxSplits = 16;
static_assert(kTailMaxSplitsPlan <= kTailMaxSplits, "the reduce holds every split");
constexpr int kTailReduceWaves = 4;
// 1024 workgroups: at the MoE w2 size (32 tail tiles x 128 rows) one
// (tile, row) pair per wave, all loads in flight at once (256 workgroups:
// 17 us, four pairs per wave one after another)
#ifndef BI8_TAIL_REDUCE_BLOCKS
#define BI8_TAIL_REDUCE_BLOCKS 1024
#endif
constexpr int kTailReduceBlocks = BI8_TAIL_REDUCE_BLOCKS;
template <int BN, int BM>
__global__ __launch_bounds__(kTailReduceWaves * 64) void moe_tail_reduce_kernel(GemmArgs p) {
    const int64_t tiles_m = moe_tiles_m<BM>(p);
    const TailPlan tp = tail_plan(tiles_m * p.tiles_n, p.KB);
    if (tp.splits <= 1) return;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kTailReduceWaves + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * kTailReduceWaves;
    for (int64_t pair = wave; pair < tp.tail * BM; pair += waves) {
        const int64_t i = pair / BM;
        const int r = (int)(pair - i * BM);
        Tile t;
        if (!tile_at<BN, BM, true, kGroupM>(p, tp.full + i, tiles_m, t)) continue;
        if (r >= t.rows) continue;
        const float *slots = p.partial + i * tp.splits * (BM * BN) + (int64_t)r * BN;
        uint16_t *yrow = p.y + (t.m0 + r) * p.N;
#pragma unroll
        for (int c0 = 0; c0 < BN; c0 += 256) {
            const int c = c0 + 4 * lane;
            const int64_t n = t.n0 + c;
            if (n >= p.N) continue;
            f32x4 part[kTailMaxSplits];
#pragma unroll
            for (int z = 0; z < kTailMaxSplits; ++z)
                if (z < tp.splits) part[z] = *reinterpret_cast<const f32x4 *>(slots + (int64_t)z * (BM * BN) + c);
            f32x4 acc = part[0];
#pragma unroll
            for (int z = 1; z < kTailMaxSplits; ++z)
                if (z < tp.splits) acc += part[z];
            if (p.wide_store && n + 4 <= p.N) {
                *reinterpret_cast<uint2 *>(yrow + n) =
                    make_uint2(f32x2_to_bf16x2_bits(acc[0], acc[1]), f32x2_to_bf16x2_bits(acc[2], acc[3]));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < p.N) yrow[n + e] = (uint16_t)(f32x2_to_bf16x2_bits(acc[e], 0.0f) & 0xFFFFu);
            }
        }
    }
}

template <bool MOE, bool SILU = false>
hipError_t launch_wide(GemmArgs p, hipStream_t stream) {
    const int64_t total = p.tiles_m * p.tiles_n;
    if (total <= 0) return hipSuccess;
    if (total > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_wide_kernel<MOE, SILU>), dim3((unsigned)total), dim3(WideCfg::kThreads), 0,
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
    p.acc_bias = kAccBias;
    return p;
}

}  // namespace

// Split K for grids of few tiles.  A 128 x 64 grid of at most one tile per
// CU runs one workgroup per CU, walking all of K one block after another at
// a pace set by latency; splitting K gives each CU several shorter, independent
// runs.  Only when the problem would take the 128 x 64 kernel with such a
// grid and K holds at least 8 blocks per split.
int32_t splitk_splits(int64_t M, int64_t N, int64_t K) {
    if (K % 16 != 0 || select_gemm_path(M, N, K) != GemmPath::kTile128x64) return 1;
    const int64_t tiles = ((M + 63) / 64) * ((N + 127) / 128);
    const int64_t KB = (K + kBlock - 1) / kBlock;
    if (tiles > 256 || M * N > kSplitKMaxOutputs) return 1;
    int64_t s = kSplitKTarget / tiles;   // all splits of all tiles in one round
    if (s > KB / 8) s = KB / 8;
    if (s > 16) s = 16;
    if (s < 2) return 1;
    const int64_t per = (KB + s - 1) / s;
    return (int32_t)((KB + per - 1) / per);   // no empty split
}

int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int32_t s = splitk_splits(M, N, K);
    return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

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
// from the mean segment length.  The 256 x 256 kernel needs four full rounds
// of the chip's CUs: with fewer its coarse tiles leave a large last round, and
// the 256 x 128 ping-pong kernel is faster (measured: the MoE w2 projection,
// 544 wide tiles, 707 -> 650 us; w13, 3808 wide tiles, the two within 1 %).
GemmPath select_moe_gemm_path(int64_t R, int64_t N, int64_t K, int32_t E) {
    (void)K;
    const int64_t rows_per_expert = E > 0 ? R / E : R;
    const int64_t wide_tiles = (int64_t)E * ((rows_per_expert + 255) / 256) * ((N + 255) / 256);
    return wide_tiles >= 1024 ? GemmPath::kTile256x256 : GemmPath::kTile256x128;
}

hipError_t launch_gemm(GemmPath path, const int8_t *xq, const float *xs, const int8_t *w,
                       const float *ws, const uint16_t *bias, uint16_t *y, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream) {
    GemmArgs p = make_args(xq, xs, w, ws, bias, y, M, N, K);
    if (K % 16 != 0) {   // rows at any byte: one kernel for every shape
        if (path != GemmPath::kAuto) return hipErrorInvalidValue;
        return launch_skinny<false, true>(p, stream);
    }
    if (path == GemmPath::kAuto) path = select_gemm_path(M, N, K);
    switch (path) {
        case GemmPath::kSkinny: {
            if (M > kSkinnyMaxM) return hipErrorInvalidValue;
            return launch_skinny<false, false>(p, stream);
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

hipError_t launch_gemm_ws(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                          const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K, float *workspace,
                          int64_t workspace_bytes, hipStream_t stream) {
    const int32_t splits = splitk_splits(M, N, K);
    if (splits < 2 || !workspace || workspace_bytes < splitk_workspace_bytes(M, N, K))
        return launch_gemm(GemmPath::kAuto, xq, xs, w, ws, bias, y, M, N, K, stream);
    GemmArgs p = make_args(xq, xs, w, ws, bias, y, M, N, K);
    p.tiles_m = (M + 63) / 64;
    p.tiles_n = (N + 127) / 128;
    p.partial = workspace;
    p.kb_per_split = (p.KB + splits - 1) / splits;
    p.wide_store = N % 4 == 0;   // the workspace is 16-byte aligned: fp32 rows take 16-byte stores
    hipError_t e = kSplitKStages == 4 ? launch_tiled<4, 2, 1, 1, false, false, 4, true>(p, stream, splits)
                                      : launch_tiled<4, 2, 1, 1, false, true, 3, true>(p, stream, splits);
    if (e != hipSuccess) return e;
    const bool vec = N % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
    const int64_t threads = vec ? (M * N) / 4 : M * N;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFFll) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, workspace, splits,
                           M, N, bias, y);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, workspace,
                           splits, M, N, bias, y);
    return hipGetLastError();
}

hipError_t launch_gemm_per_channel(const int8_t *xq, const float *xs, const int8_t *w, const float *ws,
                                   const uint16_t *bias, uint16_t *y, int64_t M, int64_t N, int64_t K,
                                   hipStream_t stream) {
    GemmArgs p = make_args(xq, xs, w, ws, bias, y, M, N, K);
    p.NB = N;   // one scale per weight row
    if (K % 16 != 0) return launch_skinny<true, true>(p, stream);   // rows at any byte
    if (use_skinny(M, N, true)) return launch_skinny<true, false>(p, stream);
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

int64_t moe_gemm_workspace_bytes(int64_t R, int64_t N, int64_t K, int32_t E) {
    if (select_moe_gemm_path(R, N, K, E) != GemmPath::kTile256x128) return 0;
    return kTailRound * 256 * 128 * (int64_t)sizeof(float);   // one slot per unit of one round
}

hipError_t launch_moe_gemm_ws(const int8_t *xq, const float *xs, const int32_t *offsets, const int8_t *w,
                              const float *ws, uint16_t *y, int64_t R, int64_t N, int64_t K, int32_t E,
                              float *workspace, int64_t workspace_bytes, hipStream_t stream) {
    const int64_t need = moe_gemm_workspace_bytes(R, N, K, E);
    if (need == 0 || !workspace || workspace_bytes < need)
        return launch_moe_gemm(GemmPath::kAuto, xq, xs, offsets, w, ws, y, R, N, K, E, stream);
    GemmArgs p = make_args(xq, xs, w, ws, nullptr, y, R, N, K);
    p.offsets = offsets;
    p.E = E;
    p.partial = workspace;
    p.tiles_m = (R + 127) / 128 + E;   // >= sum over experts of ceil(rows_e / 128)
    p.tiles_n = (N + 255) / 256;
    // every tile of that bound, plus one round for the split units
    const int64_t grid = p.tiles_m * p.tiles_n + kTailRound;
    if (grid > 0x7FFFFFFFll) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_tiled_kernel<4, 2, 2, 2, true, true, 3, true>), dim3((unsigned)grid), dim3(512), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((moe_tail_reduce_kernel<256, 128>), dim3((unsigned)kTailReduceBlocks),
                       dim3(kTailReduceWaves * 64), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_moe_gemm_silu_quant(const int8_t *xq, const float *xs, const int32_t *offsets, const int8_t *w13,
                                      const float *ws13, int8_t *aq, float *as, int64_t R, int64_t I, int64_t K,
                                      int32_t E, hipStream_t stream) {
    if (I % kBlock != 0) return hipErrorInvalidValue;
    GemmArgs p = make_args(xq, xs, w13, ws13, nullptr, nullptr, R, 2 * I, K);
    p.offsets = offsets;
    p.E = E;
    p.aq = aq;
    p.as = as;
    p.I = I;
    p.tiles_m = (R + 255) / 256 + E;   // >= sum over experts of ceil(rows_e / 256)
    p.tiles_n = I / kBlock;
    return launch_wide<true, true>(p, stream);
}

}  // namespace bi8
