// Prefill W4A16 GEMM (m > 64) for gfx950: a compute-bound tile GEMM on the
// fp16 matrix cores with the INT4 weights dequantized on the fly.
//
// Same result definition as the decode kernel (GLM-130B paper card,
// "Method"; paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s"):
// y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r]), fp32 accumulation,
// optional fused GeGLU (paper card "Hyperparameters"; paperlayer.ai B.3).
//
// Tiling.  A 256-thread workgroup computes a (4 x 16 WN weight rows) x
// (16 WT tokens) output tile over 128-wide reduction steps.  The four
// wavefronts split the rows: wave w owns WN groups of 16 rows and all WT
// token blocks, i.e. WN x WT MFMA 16x16 tiles.  Dequantizing the weights
// is the main VALU cost, so each dequantized A operand feeds WT MFMAs and
// each activation B operand read from LDS feeds WN MFMAs.
//  * Activations: the (16 WT) x 128 fp16 step tile goes global -> LDS by
//    LDS DMA (buffer loads that write LDS directly: no registers, no VALU),
//    double-buffered so the next step's copy overlaps this step's MFMAs.
//    Each token row is 256 bytes = 16 pieces of 16 bytes; piece p of row r
//    is stored at piece p ^ (r mod 16), so the 16 lanes that read one
//    operand column (16 rows, one piece) hit 16 distinct bank groups.
//  * Weights: each lane loads its 16 packed bytes per row group straight
//    into registers (one dwordx4, prefetched a step ahead, through the
//    caches: the token tiles of one row block run side by side and share
//    it) and dequantizes
//    them into the MFMA A operand: the fp16 weight tile never exists in
//    memory.  The scale is applied once per output in the epilogue.
//  * All loads are unconditional range-checked buffer loads at a per-lane
//    constant offset plus a wave-uniform step.  Rows and tokens past the
//    end are clamped to the last one (their results are never stored) and
//    steps past the end read zeros.  The step loop is unrolled twice over
//    two weight register sets, so no register copy forces a load to retire
//    early.
//  * INT8 codes (the W8A16 variant, one byte per code) take two 16-byte
//    weight loads per lane and row group per step and dequantize with
//    dequant8_i8; everything else is shared.
//  * KH = 2 splits the reduction inside the workgroup for grids of about
//    one tile per CU or fewer: 512 threads, the first four wavefronts take
//    the even 128-wide steps and the other four the odd ones, each group
//    with its own activation tiles; at the end the second group's partial
//    sums pass through LDS and the first group adds them (a fixed order,
//    so results are deterministic) before its epilogue.  Twice the
//    wavefronts per tile without smaller tiles, so each weight is still
//    dequantized once per 64 or 128 tokens.
#include "common.hpp"

#include <math.h>

namespace w4a16 {

constexpr int kPBK = 128;                 // reduction step
constexpr int kPRowBytes = 2 * kPBK;      // bytes of one token row per step
constexpr int kPThreads = 256;

template <int WN, int WT, bool EVEN, bool GEGLU, bool TILED, int CB, bool ZP, int KH>
__global__ __launch_bounds__(kPThreads * KH, KH == 1 ? 2 : 1) void prefill_kernel(const uint16_t *__restrict__ x,
                                                            int64_t m, int64_t k,
                                                            const uint8_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            int64_t n_out,
                                                            const uint16_t *__restrict__ bias,
                                                            const uint8_t *__restrict__ zeros,
                                                            uint16_t *__restrict__ y,
                                                            int tiles_m)
{
    static_assert(!GEGLU || WN % 2 == 0, "GeGLU pairs gate and value row groups");
    static_assert(CB == 4 || CB == 8, "INT4 or INT8 codes");
    static_assert(!ZP || CB == 4, "zero points are an INT4 variant");
    constexpr int WP = CB / 4;                        // 16-byte weight pieces per lane and step
    constexpr int BM = 16 * WT;                       // tokens per tile
    constexpr int NO = GEGLU ? WN / 2 : WN;           // output row groups per wave
    constexpr int kStepBytes = BM * kPRowBytes;       // activation tile of one step
    constexpr int XC = kStepBytes / (4 * 1024);       // 1 KB DMA loads per wave per step
    static_assert(XC * 4 * 1024 == kStepBytes, "activation tile must split into 1 KB loads");
    __shared__ __attribute__((aligned(1024))) uint8_t xs[KH][2][kStepBytes];

    const int lane = threadIdx.x % kWave;
    // uniform: the DMA destinations and row offsets stay in scalar registers
    static_assert(KH == 1 || KH == 2, "one or two reduction parts");
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int kh = wave_all / 4;                      // reduction part: steps kh, kh + KH, ...
    const int wave = wave_all % 4;                    // row slot of the tile
    // steps per reduction part; a part's step past the end reads zeros
    const int64_t nls = (((k + kPBK - 1) / kPBK) + KH - 1) / KH;
    const int r16 = lane % 16;
    const int g = lane / 16;

    const int tile_m = blockIdx.x % tiles_m;
    const int64_t tile_n = blockIdx.x / tiles_m;
    const int64_t m0 = (int64_t)tile_m * BM;
    const int64_t o0 = (tile_n * 4 + wave) * (16 * NO);   // first output of this wave
    const int64_t kb = k * CB / 8;                    // bytes of a row-major row
    const int64_t kt = (k + 127) / 128;
    const int64_t nsteps = (k + kPBK - 1) / kPBK;
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, code_weight_bytes(CB, TILED, rows, k));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, m * k * 2);
    const uint32_t k32 = (uint32_t)k;

    // per-lane constant part of the weight offsets; row group j is output
    // group j % NO, and for GeGLU j >= NO is the value partner of gate j - NO
    uint32_t wbase[WN];
    ZBias zb[ZP ? WN : 1];                            // zero-point subtrahends of this lane's rows
#pragma unroll
    for (int j = 0; j < WN; ++j) {
        int64_t o = o0 + 16 * (j % NO) + r16;
        if (o >= n_out)
            o = n_out - 1;
        const int64_t row = j >= NO ? n_out + o : o;
        wbase[j] = TILED ? (uint32_t)((row >> 4) * kt * 1024 * WP + 16 * lane)
                         : (uint32_t)(row * kb + 16 * WP * g);
        if constexpr (ZP)
            zb[j] = make_zbias(zeros[row]);
    }
    // DMA load i of this wave fills LDS bytes [1024 c, 1024 c + 1024) of the
    // step tile, c = XC wave + i: lane l writes token row 4 c + l / 16 at
    // stored piece l % 16, i.e. it fetches logical piece (l % 16) ^ (row % 16)
    uint32_t xbase[XC], xcol[XC];
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int row = 4 * (XC * wave + i) + lane / 16;
        const int piece = (lane % 16) ^ (row % 16);
        int64_t mi = m0 + row;
        if (mi >= m)
            mi = m - 1;
        xcol[i] = 8 * piece;
        xbase[i] = (uint32_t)(mi * k * 2 + 16 * piece);
    }
    // LDS read offsets of this lane's B operand pieces: token row r16 of
    // each block, logical piece 4 g + t
    uint32_t rdoff[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        rdoff[t] = r16 * kPRowBytes + 16 * ((4 * g + t) ^ r16);

    float4v acc[WN][WT];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int b = 0; b < WT; ++b)
            acc[j][b] = float4v{0.f, 0.f, 0.f, 0.f};

    // Offsets below 2^31 plus kOutOfRange stay below 2^32 and out of range,
    // so a step past the end reads zeros.
    auto load_x = [&](int64_t ls, int buf) {
        const int64_t s = ls * KH + kh;
        const uint32_t step = s < nsteps ? (uint32_t)s * kPRowBytes : kOutOfRange;
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            uint32_t off = xbase[i] + step;
            if (!EVEN && (uint32_t)s * kPBK + xcol[i] >= k32)
                off = kOutOfRange;
            buf_load16_lds(xrs, off, &xs[kh][buf][1024 * (XC * wave + i)]);
        }
    };
    // INT8 codes take two 16-byte loads per row group: the lane's next 16
    // bytes (row-major) or the tile's second KB (prepacked).
    auto load_w = [&](int64_t ls, u32x4(&wd)[WN][WP]) {
        const int64_t s = ls * KH + kh;
        const uint32_t u = (uint32_t)s * kPBK;
        const uint32_t step = s < nsteps ? (TILED ? (uint32_t)s * 1024u * WP : u * CB / 8) : kOutOfRange;
#pragma unroll
        for (int j = 0; j < WN; ++j) {
            uint32_t off = wbase[j] + step;
            if (!EVEN && !TILED && u + 32 * g >= k32)
                off = kOutOfRange;
#pragma unroll
            for (int h = 0; h < WP; ++h)
                wd[j][h] = buf_load16(wrs, off + h * (TILED ? 1024u : 16u));
        }
    };
    // MFMA t of a step covers, for lane group g, reduction indices
    // 32 g + 8 t .. + 7 of the step on both operands.  The WN dequantized
    // A operands stay live while the B operands stream through.
    auto compute = [&](int buf, const u32x4(&wd)[WN][WP]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 a[WN];
#pragma unroll
            for (int j = 0; j < WN; ++j) {
                if constexpr (ZP)
                    a[j] = dequant8_zp_of<TILED>(wd[j][0][t], zb[j]);
                else if constexpr (CB == 4)
                    a[j] = dequant8_of<TILED>(wd[j][0][t]);
                else
                    a[j] = dequant8_i8_of<TILED>(wd[j][t / 2][2 * (t % 2)], wd[j][t / 2][2 * (t % 2) + 1]);
            }
#pragma unroll
            for (int b = 0; b < WT; ++b) {
                const half8 bx = as_half8(*reinterpret_cast<const u32x4 *>(
                    &xs[kh][buf][rdoff[t] + 16 * kPRowBytes * b]));
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[j][b] = mfma16x16x32(a[j], bx, acc[j][b]);
            }
        }
    };
    // Each step issues its activation DMA, then its WN weight loads, kept
    // in that order and at the top of the step by scheduling barriers (the
    // compiler would otherwise sink the weight loads to the end of the
    // step, next to their first use, and expose their whole latency).
    // Loads retire in order, so waiting until at most WN are outstanding
    // means this wave's DMA writes have landed; the barrier then hands the
    // buffer to the other waves while the weight loads stay in flight.
    // The fences order only LDS accesses around the barrier.
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(WN * WP));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // two register sets for the weights, used alternately (the loop is
    // unrolled twice so no set is ever copied)
    u32x4 wa[WN][WP], wb[WN][WP];
    load_x(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(0, wa);
    publish();
    for (int64_t s = 0;;) {
        load_x(s + 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s + 1, wb);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, wa);
        publish();
        if (++s >= nls)
            break;
        load_x(s + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(s + 1, wa);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, wb);
        publish();
        if (++s >= nls)
            break;
    }
    if constexpr (KH > 1) {
        // partial sums of reduction parts 1..KH-1 -> LDS (no wave reads the
        // activation tiles after the last barrier); part 0 adds them in order
        constexpr int kSlot = WN * WT * 4 * kWave;        // floats per wave
        static_assert((KH - 1) * 4 * kSlot * 4 <= (int)sizeof(xs), "partials fit the tiles' LDS");
        float *red = reinterpret_cast<float *>(&xs[0][0][0]);
        if (kh > 0) {
#pragma unroll
            for (int j = 0; j < WN; ++j)
#pragma unroll
                for (int b = 0; b < WT; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        red[((kh - 1) * 4 + wave) * kSlot + ((j * WT + b) * kWave + lane) * 4 + i] = acc[j][b][i];
        }
        __syncthreads();
        if (kh > 0)
            return;
#pragma unroll
        for (int q = 1; q < KH; ++q)
#pragma unroll
            for (int j = 0; j < WN; ++j)
#pragma unroll
                for (int b = 0; b < WT; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j][b][i] += red[((q - 1) * 4 + wave) * kSlot + ((j * WT + b) * kWave + lane) * 4 + i];
    }

    // epilogue: lane holds D[4 g + i][r16] of tile (j, b), i.e. outputs
    // 16 j + 4 g + i of the wave for token 16 b + r16: four consecutive
    // outputs, stored as one 8-byte write when all are in range and aligned
    const bool vec = (n_out % 4) == 0;
#pragma unroll
    for (int b = 0; b < WT; ++b) {
        const int64_t mi = m0 + 16 * b + r16;
        if (mi >= m)
            continue;
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int64_t ob = o0 + 16 * j + 4 * g;
            if (ob >= n_out)
                continue;
            uint16_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t o = ob + i < n_out ? ob + i : n_out - 1;
                // s acc + bias with one fp32 rounding (bias 0 when absent),
                // as in the decode kernel
                float v;
                if (GEGLU) {
                    const float a = __builtin_fmaf(acc[j][b][i], half_bits_to_float(scales[o]),
                                                   bias ? half_bits_to_float(bias[o]) : 0.0f);
                    const float bv = __builtin_fmaf(acc[j + NO][b][i], half_bits_to_float(scales[n_out + o]),
                                                    bias ? half_bits_to_float(bias[n_out + o]) : 0.0f);
                    v = gelu_erf(a) * bv;
                } else {
                    v = __builtin_fmaf(acc[j][b][i], half_bits_to_float(scales[o]),
                                       bias ? half_bits_to_float(bias[o]) : 0.0f);
                }
                h[i] = output_half_bits(v);
            }
            uint16_t *dst = y + mi * n_out + ob;
            if (vec && ob + 3 < n_out) {
                uint2 pk;
                pk.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                pk.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                *reinterpret_cast<uint2 *>(dst) = pk;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (ob + i < n_out)
                        dst[i] = h[i];
            }
        }
    }
}

template <int WN, int WT, bool GEGLU, bool TILED, int CB, bool ZP, int KH = 1>
static hipError_t launch_prefill_t(const void *x, int64_t m, int64_t k, const void *packed,
                                   const void *scales, int64_t n_out, const void *bias,
                                   const void *zeros, void *y, hipStream_t stream)
{
    constexpr int out_per = 4 * 16 * (GEGLU ? WN / 2 : WN);
    const int64_t tiles_n = (n_out + out_per - 1) / out_per;
    const int64_t tiles_m = (m + 16 * WT - 1) / (16 * WT);
    const int64_t grid = tiles_n * tiles_m;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const uint8_t *pp = static_cast<const uint8_t *>(packed);
    const uint16_t *sp = static_cast<const uint16_t *>(scales);
    const uint16_t *bp = static_cast<const uint16_t *>(bias);
    const uint8_t *zp = static_cast<const uint8_t *>(zeros);
    uint16_t *yp = static_cast<uint16_t *>(y);
#define W4_PREFILL(EV)                                                                            \
    hipLaunchKernelGGL((prefill_kernel<WN, WT, EV, GEGLU, TILED, CB, ZP, KH>), dim3((unsigned)grid), \
                       dim3(kPThreads * KH), 0, stream, xp, m, k, pp, sp, n_out, bp, zp, yp, (int)tiles_m)
    if (k % kPBK == 0)
        W4_PREFILL(true);
    else
        W4_PREFILL(false);
#undef W4_PREFILL
    return hipGetLastError();
}

// Fraction of the last wave of workgroups that is filled, two resident
// workgroups per compute unit (64 KB of LDS each).
static double wave_fill(int64_t grid, int64_t slots)
{
    const int64_t waves = (grid + slots - 1) / slots;
    return (double)grid / (double)(waves * slots);
}

static int64_t compute_units()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

// Small plain grids: the tile shape (and reduction split) with the least
// modelled time.  Shape i has tiles of 64 WN rows x 16 WT tokens, `slots`
// workgroups resident per CU (from its registers and LDS) and a relative
// throughput `rate`.  A grid of g tiles runs full = g / (slots cus) rounds
// of `slots` concurrent tiles per CU and a last round of r = ceil(rem /
// cus); j concurrent tiles on a CU take j^0.7 single-tile times (a CU's
// throughput grows as j^0.3 with more resident tiles), so the modelled time
// is (full slots^0.7 + r^0.7) 64 WN 16 WT / rate.  The rates and the
// exponent were fitted to 166 timings of every shape at the GLM-130B widths
// and their 2-, 4- and 8-way shards (n = 4608 ... 65536, k = 3072 ... 32768,
// m = 129 ... 1024, every grid of this branch): the chosen shape came within
// 0.35% of the fastest on average, where fixed thresholds were 4.6% off
// (and up to 21%: the 4-way QKV shard 9216 x 12288 at m = 129 ... 192 runs
// 52 us on split 128 x 64 tiles against 66 us on 192 x 64 ones).
struct SmallTile {
    int wn, wt, kh, slots;
    double rate;
};
// (192 x 128 tiles were fitted too, rate 0.934, but are never the least
// time on this branch; the split 192 x 128 tiles are chosen before it.)
constexpr SmallTile kSmallTiles[] = {{3, 4, 1, 4, 0.809}, {4, 4, 1, 3, 0.899}, {4, 8, 1, 2, 1.0},
                                     {3, 4, 2, 2, 0.906}, {2, 4, 2, 2, 0.835}};

static int small_grid_tile(int64_t m, int64_t n_out, int64_t cus)
{
    int best = 0;
    double best_t = 0.0;
    for (int i = 0; i < (int)(sizeof kSmallTiles / sizeof kSmallTiles[0]); ++i) {
        const SmallTile &t = kSmallTiles[i];
        const int64_t rows = 64 * t.wn, tokens = 16 * t.wt;
        const int64_t g = ((n_out + rows - 1) / rows) * ((m + tokens - 1) / tokens);
        const int64_t full = g / (t.slots * cus), rem = g - full * t.slots * cus;
        const int64_t r = (rem + cus - 1) / cus;
        const double units = (double)full * pow((double)t.slots, 0.7) + (r ? pow((double)r, 0.7) : 0.0);
        const double time = units * (double)(rows * tokens) / t.rate;
        if (i == 0 || time < best_t) {
            best = i;
            best_t = time;
        }
    }
    return best;
}

template <bool GEGLU, bool TILED, int CB, bool ZP>
static hipError_t launch_prefill_layout(const void *x, int64_t m, int64_t k, const void *packed,
                                        const void *scales, int64_t n_out, const void *bias,
                                        const void *zeros, void *y, hipStream_t stream)
{
    // Tile shape from the grid of the largest tile (4 x 16 x 4 rows x 128
    // tokens; GeGLU 128 outputs x 128 tokens), measured at the GLM-130B
    // widths for m = 128 ... 2048:
    //  * a plain grid of at most about two such tiles per CU that does not
    //    fill a whole wave of workgroups (two per CU) leaves CUs idle or
    //    thinly used: with k >= 8192 and about one 192 x 128 tile per CU
    //    (7/8 to 1) it takes those tiles with the reduction split over two
    //    halves of a 512-thread workgroup (attention-out 12288 x 12288 at
    //    m = 512: 131.5-131.8 against 136.0-136.2 us split 192 x 64;
    //    FFN-down 12288 x 32768 at m = 512: 334-342 against 360-376 us),
    //    otherwise the shape of least modelled time (small_grid_tile:
    //    192 or 256 rows x 64 or 128 tokens, or 192 or 128 rows x 64 tokens
    //    with the reduction split);
    //  * larger plain grids keep 128-token tiles unless 64-token tiles fill
    //    the last wave of workgroups much better (k <= 16384) and the
    //    128-token grid's last wave would leave at least half the CUs idle
    //    (QKV at m = 1024: 736 against 746 us), or the reduction is short
    //    (k < 4096).  A last wave that gives each CU one workgroup costs
    //    little, since those workgroups run with the CU to themselves:
    //    attention-out 12288 x 12288 at m = 2048 runs 470-476 us on
    //    128-token tiles against 484-486 us on 64-token tiles, QKV at
    //    m = 1536 1037-1040 against 1089-1091 us;
    //  * GeGLU grids of at most one 128 x 128 tile per CU take 64-output
    //    tiles, 128 tokens wide when that grid still gives two per CU (FFN-up
    //    65536 x 12288 at m = 128: 188.9 against 200.0 us for 64 x 64 tiles;
    //    its 4-way shard 16384 x 12288 at m = 512: 177.4 against 187.6 us);
    //  * larger GeGLU grids take 128 x 128 tiles, or 128 outputs x 64 tokens
    //    where 128-token tiles would pad half a tile more and the 64-token
    //    grid fits one wave at three per CU (FFN-up at m = 192: 268.6
    //    against 326.4 us); the split reduction gains nothing for GeGLU.
    //  * INT8 codes need a second weight register set per row group, so
    //    their large tiles keep 128 tokens with one row group fewer per
    //    wave: 192 rows (GeGLU: 64 outputs) x 128 tokens, 188-204 VGPRs
    //    and no spill.  Against 256 x 64 tiles at m = 2048: attention-out
    //    498 against 559 us, plain FFN-up 2698 against 3046 us, GeGLU
    //    FFN-up 2929 against 3060 us.  256 x 128 tiles (250 VGPRs, the same
    //    two waves per SIMD) time the same; split-reduction tiles are
    //    slower.
    constexpr int out_per = 4 * 16 * (GEGLU ? 2 : 4);
    const int64_t tiles_n = (n_out + out_per - 1) / out_per;
    const int64_t cus = compute_units();
    const int64_t g48 = tiles_n * ((m + 127) / 128);
    if constexpr (CB == 8) {
        if constexpr (GEGLU) {
            if (g48 <= cus)
                return launch_prefill_t<2, 4, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
            return launch_prefill_t<2, 8, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
        } else {
            if (4 * g48 <= 9 * cus && wave_fill(g48, 2 * cus) < 0.9)
                return launch_prefill_t<3, 4, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
            return launch_prefill_t<3, 8, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
        }
    } else if constexpr (GEGLU) {
        const int64_t tm8 = (m + 127) / 128, tm4 = (m + 63) / 64;
        if (g48 <= cus) {
            // 64-output tiles; 128 tokens when that grid still gives two per CU
            if (((n_out + 63) / 64) * tm8 >= 2 * cus)
                return launch_prefill_t<2, 8, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
            return launch_prefill_t<2, 4, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
        }
        // 64-token tiles when 128-token ones would pad half a tile more and
        // the 64-token grid fits one wave at three per CU
        if (tm8 * 128 - tm4 * 64 >= 64 && tiles_n * tm4 <= 3 * cus)
            return launch_prefill_t<4, 4, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
        return launch_prefill_t<4, 8, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
    } else {
        const int64_t slots = 2 * cus;
        const double fill8 = wave_fill(g48, slots);
        if (4 * g48 <= 9 * cus && fill8 < 0.9) {
            // small grids: about one 192 x 128 tile per CU with a long
            // reduction takes those tiles with the reduction split; other
            // small grids take the shape of least modelled time
            const int64_t g38 = ((n_out + 191) / 192) * ((m + 127) / 128);
            if (k >= 8192 && 8 * g38 >= 7 * cus && g38 <= cus)
                return launch_prefill_t<3, 8, GEGLU, TILED, CB, ZP, 2>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
#define W4_SMALL(I, WN, WT, KH)                                                                    \
    case I:                                                                                        \
        return launch_prefill_t<WN, WT, GEGLU, TILED, CB, ZP, KH>(x, m, k, packed, scales, n_out, bias, \
                                                                  zeros, y, stream)
            switch (small_grid_tile(m, n_out, cus)) {
                W4_SMALL(0, 3, 4, 1);
                W4_SMALL(1, 4, 4, 1);
                W4_SMALL(2, 4, 8, 1);
                W4_SMALL(3, 3, 4, 2);
                default:
                W4_SMALL(4, 2, 4, 2);
            }
#undef W4_SMALL
        }
        const double fill4 = wave_fill(tiles_n * ((m + 63) / 64), slots);
        const int64_t last = g48 % slots;             // workgroups of a partial last wave
        if (k <= 16384 && fill4 > fill8 + 0.1 && ((last > 0 && 2 * last <= cus) || k < 4096))
            return launch_prefill_t<4, 4, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
        return launch_prefill_t<4, 8, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, bias, zeros, y, stream);
    }
}

hipError_t launch_prefill(const void *x, int64_t m, int64_t k, const void *packed,
                          const void *scales, int64_t n_out, const void *bias, const void *zeros,
                          void *y, bool geglu, bool tiled, int cb, hipStream_t stream)
{
#define W4_PLAYOUT(G, T, C, Z)                                                                    \
    launch_prefill_layout<G, T, C, Z>(x, m, k, packed, scales, n_out, bias, zeros, y, stream)
    if (cb == 8) {
        if (geglu)
            return tiled ? W4_PLAYOUT(true, true, 8, false) : W4_PLAYOUT(true, false, 8, false);
        return tiled ? W4_PLAYOUT(false, true, 8, false) : W4_PLAYOUT(false, false, 8, false);
    }
    if (zeros) {
        if (geglu)
            return tiled ? W4_PLAYOUT(true, true, 4, true) : W4_PLAYOUT(true, false, 4, true);
        return tiled ? W4_PLAYOUT(false, true, 4, true) : W4_PLAYOUT(false, false, 4, true);
    }
    if (geglu)
        return tiled ? W4_PLAYOUT(true, true, 4, false) : W4_PLAYOUT(true, false, 4, false);
    return tiled ? W4_PLAYOUT(false, true, 4, false) : W4_PLAYOUT(false, false, 4, false);
#undef W4_PLAYOUT
}

}  // namespace w4a16
