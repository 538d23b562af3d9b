// Decode W4A16 GEMV / skinny GEMM kernel template (m <= 64 tokens per launch; the library
// runs it twice for 64 < m <= 128) for gfx950.
//
// y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r])   (GLM-130B paper
// card, "Method": linear_forward with the weights turned back into FP16 at
// run time; paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s").
// At decode sizes the packed weights dominate the traffic (k/2 bytes per
// row against 2 m k bytes of activations), so the kernel is built to stream
// the weights from HBM once at full bandwidth (one template, shaped per
// token count and weight height):
//
//  * Codes become exact fp16 integers in registers (dequant8: 9 VALU ops
//    per 8 codes of the prepacked layout, 12 for the row-major one) and
//    feed v_mfma_f32_16x16x32_f16 with 16 weight rows as the
//    A operand and up to 16 tokens per MFMA as the B operand, fp32
//    accumulation.  Padding m up to 16 costs idle MFMA slots, not bytes.
//  * Every load is an unconditional range-checked buffer load (padding
//    lanes read zeros), and the main loop is unrolled over a ring of
//    register sets, so the next rounds' loads stay in flight while the
//    current round is multiplied (no register copies that would force the
//    loads to retire).
//  * The row scale is constant along the sum, so it is applied once to the
//    fp32 sum in the epilogue instead of to every weight; then the bias,
//    the optional GeGLU, and one fp16 rounding.
//  * CB = 8 instantiates the INT8 variant (W8A16: the pages' b-bit scale
//    with b = 8, one code per byte): two 16-byte weight loads per lane,
//    row group and 128 indices, dequant8_i8; everything else is shared.
#pragma once

#include "common.hpp"

namespace w4a16 {

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// Four consecutive fp16 values p[o .. o + 3] (o a multiple of 4), packed
// two per word (0 for no p); entries at or past `count` repeat entry
// count - 1 (their outputs are never stored).  `whole` says that p is 8-byte
// aligned, a fact about the whole call: then one 8-byte load serves when all
// four are in range.
__device__ __forceinline__ uint2 load4_h(const uint16_t *__restrict__ p, int o, int count, bool whole)
{
    if (!p)
        return uint2{0u, 0u};
    if (whole && o + 3 < count)
        return *reinterpret_cast<const uint2 *>(p + o);
    uint32_t h[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        h[c] = p[o + c < count ? o + c : count - 1];
    return uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// Entry i (0..3) of four packed fp16 values, as a float.
__device__ __forceinline__ float half4_at(uint2 v, int i)
{
    const uint32_t w = i < 2 ? v.x : v.y;
    return half_bits_to_float((uint16_t)((i & 1) ? w >> 16 : w & 0xFFFFu));
}

// ---------------------------------------------------------------------------
// Decode kernel (m <= 64).
//
// A wavefront owns NGW groups of 16 weight rows (for GeGLU: NGW / 2 gate
// groups and the matching value groups) and MB blocks of 16 tokens.  A
// workgroup of W wavefronts (4 to 16) holds RG such row sets; the KS =
// W / RG wavefronts of a row set split the reduction into interleaved
// chunks of 128 KU indices.  A wavefront streams its rows chunk by chunk (KU 16-byte
// pieces per lane per row group), with a ring of D register sets so the
// pieces of the next D - 1 chunks are in flight while the current one is
// multiplied.  Each dequantized A operand feeds MB MFMAs (one per token
// block), and each activation operand read from LDS feeds NGW MFMAs.
//
// The activation chunks of a round (KS chunks, MR x 128 KU fp16 each; MR =
// m rounded up to 4, 8 or 16 for one block, 16 MB otherwise) are loaded
// once per workgroup and double-buffered in LDS, one barrier per round;
// the RG wavefronts that work on the same chunk share it.  Each round's activation loads are
// issued before its weight loads: vector loads retire in order, so waiting
// for the activations does not wait for the weights.  Partial sums of the
// KS wavefronts of a row set meet in LDS in a fixed order.
//
// The dequantization is the bulk of the VALU work, so
// everything else is kept off the VALU: every lane's load offset is a
// per-lane constant plus a wave-uniform step.  Rows past the end are
// clamped to the last row and tokens past m to token m - 1 (they only feed
// MFMA rows and columns that are never stored); a chunk past the end gets
// the out-of-range step, so its loads return zeros.  EVEN (k a multiple of
// the 128 KU KS-index round) needs no per-lane reduction-index checks; the
// general instantiation adds them for a ragged last round.
//
// TILED selects the prepacked weight layout (w4a16_prepack): each 16-row x
// 128-index tile is one contiguous 1 KB block in lane order, so a
// wavefront reads KU KB of consecutive memory per chunk and row group
// instead of 16 row segments of 64 KU bytes.
// ---------------------------------------------------------------------------
template <int MB, int MR>
struct TokenTile {
    static_assert(MB == 1 ? (MR == 4 || MR == 8 || MR == 16) : MR == 16 * MB, "token rows");
};

template <int KU, int RG, int W, int D, int MB, int MR, int NGW, bool EVEN, bool GEGLU, bool TILED,
          int CB, bool ZP>
__global__ __launch_bounds__(W * kWave) void decode_kernel(
    const uint16_t *__restrict__ x, int m, int64_t k, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, int64_t n_out, const uint16_t *__restrict__ bias,
    const uint8_t *__restrict__ zeros, uint16_t *__restrict__ y)
{
    (void)TokenTile<MB, MR>{};
    static_assert(!GEGLU || NGW % 2 == 0, "GeGLU pairs gate and value row groups");
    static_assert(W % RG == 0, "row sets split the wavefronts evenly");
    static_assert(CB == 4 || CB == 8, "INT4 or INT8 codes");
    static_assert(!ZP || CB == 4, "zero points are an INT4 variant");
    constexpr int KS = W / RG;
    constexpr int WP = CB / 4;                // 16-byte weight pieces per lane, row group and 128 indices
    static_assert(NGW * KU * WP * (D - 1) <= 63, "outstanding weight loads fit the vmcnt counter");
    constexpr int KC = 128 * KU;              // reduction indices per chunk
    constexpr int RP = KC / 8;                // 16-byte pieces per activation row per chunk
    // 16 or more token rows: activations by LDS DMA into XOR-swizzled rows.
    // 4 or 8 rows: through registers into padded rows (measured faster there).
    constexpr bool XDMA = MR >= 16;
    constexpr int LD = XDMA ? KC : KC + 8;    // row stride (halves)
    constexpr int SLOT = MR * LD * 2;         // bytes of one chunk slot (MR rows)
    constexpr int STAGE = KS * SLOT;          // bytes of one round's activations
    constexpr int NCH = STAGE / 1024;         // 1 KB DMA loads per round
    constexpr int NPC = KS * MR * RP;         // 16-byte activation pieces per round
    constexpr int NXI = XDMA ? (NCH + W - 1) / W
                             : (NPC + W * kWave - 1) / (W * kWave);   // per wave / thread
    static_assert(!XDMA || NCH * 1024 == STAGE, "activation round must split into 1 KB loads");
    constexpr int CH = MB == 1 ? 2 : 1;       // independent accumulator chains per (group, block)
    constexpr int OUTW = GEGLU ? 8 * NGW : 16 * NGW;   // outputs per wave
    // LDS: the double-buffered activation chunks during the loop, the
    // partial sums of K-parts 1..KS-1 after it (one buffer, two uses)
    constexpr int kSlot = NGW * MB * kWave * 4;            // partial-sum floats per wave
    constexpr int kXBytes = 2 * STAGE;
    constexpr int kRedBytes = (KS - 1) * RG * kSlot * 4;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kXBytes > kRedBytes ? kXBytes : kRedBytes];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int rgi = wave % RG;
    const int kp = wave / RG;
    const int r16 = lane % 16;
    const int g = lane / 16;
    const int64_t o0 = ((int64_t)blockIdx.x * RG + rgi) * OUTW;   // first output of this wave
    const int64_t kb = k * CB / 8;             // bytes of a row-major row
    const int64_t kt = ceil_div(k, 128);

    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, code_weight_bytes(CB, TILED, rows, k));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (int64_t)m * k * 2);

    // Per-lane constant part of each weight load offset.  Rows past the
    // end: the prepacked layout holds zero rows there (or reads past the
    // buffer, which return zeros); the row-major one is clamped to the last
    // row (the result is never stored).
    uint32_t wbase[NGW];
    ZBias zb[ZP ? NGW : 1];                    // zero-point subtrahends of this lane's rows
#pragma unroll
    for (int j = 0; j < NGW; ++j) {
        int64_t o = o0 + 16 * (GEGLU ? j % (NGW / 2 > 0 ? NGW / 2 : 1) : j) + r16;
        if (!TILED && o >= n_out)
            o = n_out - 1;
        const int64_t row = (GEGLU && j >= NGW / 2) ? n_out + o : o;
        wbase[j] = TILED ? (uint32_t)((row >> 4) * kt * 1024 * WP + 16 * lane)
                         : (uint32_t)(row * kb + 16 * WP * g);
        if constexpr (ZP)
            zb[j] = make_zbias(row < rows ? zeros[row] : 0u);
    }
    const uint32_t k32 = (uint32_t)k;

    float4v acc[NGW][MB][CH];
#pragma unroll
    for (int j = 0; j < NGW; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int c = 0; c < CH; ++c)
                acc[j][b][c] = float4v{0.f, 0.f, 0.f, 0.f};

    const int64_t nch = ceil_div(k, KC);
    const int64_t rounds = ceil_div(nch, KS);

    // Chunk c of this wave, piece p: reduction indices c KC + 128 p + 32 g.
    // The wave-uniform step (c KC + 128 p) CB / 8 bytes (row-major) or tile
    // c KU + p (prepacked) is added to the per-lane base.  INT8 codes take
    // two 16-byte loads per piece: the lane's next 16 bytes (row-major) or
    // the tile's second KB (prepacked).
    auto load_w = [&](int64_t r, u32x4(&wd)[NGW][KU * WP]) {
        const uint32_t c = (uint32_t)(r * KS + kp);
        const bool live = c < (uint32_t)nch;
#pragma unroll
        for (int p = 0; p < KU; ++p) {
            const uint32_t u = c * KC + 128 * p;
            uint32_t step = TILED ? (c * KU + p) * 1024u * WP : u * CB / 8;
            if (!live)
                step = kOutOfRange;
#pragma unroll
            for (int j = 0; j < NGW; ++j) {
                uint32_t off = wbase[j] + step;
                if (!EVEN && !TILED && u + 32 * g >= k32)
                    off = kOutOfRange;                 // ragged last piece, row-major only
#pragma unroll
                for (int h = 0; h < WP; ++h)
                    wd[j][WP * p + h] = buf_load16_stream(wrs, off + h * (TILED ? 1024u : 16u));
            }
        }
    };
    // Activation tile of a round: KS chunk slots (one per K-part) of MR
    // token rows x KC indices, row-major; tokens past m repeat token m - 1.
    //  * XDMA: rows of 256 KU bytes; the 16-byte piece P (indices 8 P ..
    //    8 P + 7 of the chunk) of row r is stored at piece P ^ (r mod 16), so
    //    the 16 rows an MFMA B-operand read touches start at different
    //    banks.  DMA load i of this wave is the round's 1 KB load c = wave +
    //    W i; lane l fills 16-byte unit 64 c + l (whole row segments, so a
    //    load covers few cache lines).
    //  * otherwise: each thread loads pieces into registers at the top of a
    //    round and stores them into rows padded by 16 bytes at its end.
    uint32_t xbase[NXI], xcol[NXI];
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
        int slot, row, piece;
        if (XDMA) {
            const int u = 64 * (wave + W * i) + lane;      // 16-byte unit of the round
            slot = u / (MR * RP);
            row = (u % (MR * RP)) / RP;
            piece = (u % RP) ^ (row & 15);
        } else {
            // pieces are dealt round-robin; surplus threads repeat one
            // (same value, same LDS address)
            const int idx = (threadIdx.x + W * kWave * i) % NPC;
            slot = idx / RP / MR;
            row = (idx / RP) % MR;
            piece = idx % RP;
        }
        const int mi = row < m ? row : m - 1;
        xcol[i] = (uint32_t)(slot * KC + 8 * piece);       // index within the round
        xbase[i] = (uint32_t)(mi * k * 2 + 2 * xcol[i]);
    }
    u32x4 xr[XDMA ? 1 : NXI];
    // Offsets below 2^31 plus kOutOfRange stay below 2^32 and out of range.
    auto load_x = [&](int64_t r, int buf) {
        const uint32_t k0 = (uint32_t)(r * KS * KC);
        const uint32_t step = r < rounds ? 2 * k0 : kOutOfRange;
#pragma unroll
        for (int i = 0; i < NXI; ++i) {
            if (XDMA && NCH % W != 0 && wave + W * i >= NCH)
                break;
            uint32_t off = xbase[i] + step;
            if (!EVEN && k0 + xcol[i] >= k32)
                off = kOutOfRange;
            if constexpr (XDMA)
                buf_load16_lds(xrs, off, lds + buf * STAGE + 1024 * (wave + W * i));
            else
                xr[i] = buf_load16(xrs, off);
        }
    };
    auto store_x = [&](int buf) {
        if constexpr (!XDMA) {
#pragma unroll
            for (int i = 0; i < NXI; ++i) {
                const int idx = (threadIdx.x + W * kWave * i) % NPC;
                *reinterpret_cast<u32x4 *>(lds + buf * STAGE + (idx / RP / MR) * SLOT +
                                           ((idx / RP) % MR) * LD * 2 + 16 * (idx % RP)) = xr[i];
            }
        }
    };
    // XDMA: loads retire in order and each round issues its activation DMA
    // before its weight loads, so waiting until at most NGW KU loads are
    // outstanding means this wave's DMA of the next round has landed; the
    // barrier then publishes it and retires the buffer the following DMA
    // overwrites (the fences order only LDS accesses around it).
    auto publish = [&]() {
        if constexpr (XDMA) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(NGW * KU * WP));
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        } else {
            __syncthreads();
        }
    };
    const int brow = r16 < MR ? r16 : MR - 1;          // MFMA columns past MR repeat row MR - 1
    const uint8_t *xrd = lds + kp * SLOT + brow * LD * 2;
    uint32_t rdoff[4];                                 // piece 4 g + t of row brow
#pragma unroll
    for (int t = 0; t < 4; ++t)
        rdoff[t] = 16 * (XDMA ? ((4 * g + t) ^ brow) : 4 * g + t);
    auto compute = [&](int buf, const u32x4(&wd)[NGW][KU * WP]) {
#pragma unroll
        for (int p = 0; p < KU; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                half8 bx[MB];
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    bx[b] = as_half8(*reinterpret_cast<const u32x4 *>(
                        xrd + buf * STAGE + (16 * b * LD + 128 * p) * 2 + rdoff[t]));
#pragma unroll
                for (int j = 0; j < NGW; ++j) {
                    half8 a;
                    if constexpr (ZP)
                        a = dequant8_zp_of<TILED>(wd[j][p][t], zb[j]);
                    else if constexpr (CB == 4)
                        a = dequant8_of<TILED>(wd[j][p][t]);
                    else
                        a = dequant8_i8_of<TILED>(wd[j][2 * p + t / 2][2 * (t % 2)],
                                                  wd[j][2 * p + t / 2][2 * (t % 2) + 1]);
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        acc[j][b][t % CH] = mfma16x16x32(a, bx[b], acc[j][b][t % CH]);
                }
            }
    };

    // Ring of D weight register sets: round r uses set r % D, loaded D - 1
    // rounds earlier.  The round loop is unrolled U times (a multiple of D
    // and of the 2 LDS buffers) so every set has a fixed register name (no
    // copies, which would force the loads to retire early).  Scheduling barriers keep each round's loads at its
    // top, activations first: left alone, the compiler sinks them towards
    // their first use and the prefetch distance collapses.
    u32x4 wr[D][NGW][KU * WP];
    load_x(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
        load_w(i, wr[i]);
    if constexpr (XDMA)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NGW * KU * WP * (D - 1)));
    store_x(0);
    publish();
    constexpr int U = D % 2 == 0 ? D : 2 * D;
    for (int64_t r0 = 0; r0 < rounds; r0 += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t r = r0 + i;
            if (r >= rounds)
                break;
            load_x(r + 1, (i & 1) ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            load_w(r + D - 1, wr[(i + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            compute(i & 1, wr[i % D]);
            store_x((i & 1) ^ 1);
            publish();
        }
    }
    if (CH > 1) {
#pragma unroll
        for (int j = 0; j < NGW; ++j)
#pragma unroll
            for (int b = 0; b < MB; ++b)
                acc[j][b][0] += acc[j][b][CH - 1];
    }

    // The epilogue's row scales and biases: lane outputs o0 + 16 j + 4 g + i
    // (i = 0..3, consecutive), loaded once, four at a time, by the waves that
    // store.  With more than four token rows they are loaded before the
    // K-part reduction, so their latency overlaps it; with four (m <= 4,
    // where one lane in 16 or fewer stores) only the storing lanes load them,
    // after it.
    constexpr int NO = GEGLU ? NGW / 2 : NGW;   // output groups
    constexpr int NV = GEGLU ? NO : 1;          // value groups (GeGLU)
    constexpr bool EARLY = MR > 4;
    // Callers pass scales, bias and y 16-byte aligned; rows of n_out fp16
    // values keep 8-byte alignment when n_out is a multiple of 4.  Output
    // indices stay below 2^31 (n_out <= 2^30).
    const int n32 = (int)n_out;
    const bool vec = n_out % 4 == 0;
    uint2 sa[NO], ba[NO], sv[NV], bv[NV];
    auto load_epilogue = [&]() {
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int ob = (int)o0 + 16 * j + 4 * g;
            sa[j] = load4_h(scales, ob, n32, true);
            ba[j] = load4_h(bias, ob, n32, true);
            if constexpr (GEGLU) {
                sv[j] = load4_h(scales + n_out, ob, n32, vec);
                bv[j] = load4_h(bias ? bias + n_out : nullptr, ob, n32, vec);
            }
        }
    };
    if (EARLY && kp == 0)
        load_epilogue();

    if (KS > 1) {
        // partial sums of K-parts 1..KS-1 -> LDS; K-part 0 adds them in order
        float *red = reinterpret_cast<float *>(lds);
        if (kp > 0) {
#pragma unroll
            for (int j = 0; j < NGW; ++j)
#pragma unroll
                for (int b = 0; b < MB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        red[((kp - 1) * RG + rgi) * kSlot + ((j * MB + b) * kWave + lane) * 4 + i] =
                            acc[j][b][0][i];
        }
        __syncthreads();
        if (kp > 0)
            return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int j = 0; j < NGW; ++j)
#pragma unroll
                for (int b = 0; b < MB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j][b][0][i] +=
                            red[((q - 1) * RG + rgi) * kSlot + ((j * MB + b) * kWave + lane) * 4 + i];
        // With 3 or more waves per SIMD (at most 168 registers) and 12 or
        // more accumulator tiles per wave, pin the sums here: left alone, the
        // compiler sinks each add into the epilogue's per-output branches,
        // keeps every partial read live until then and spills 44 registers.
        // Smaller shapes do not spill and measure faster without the pin.
        if constexpr (W >= 12 && NGW * MB >= 12) {
#pragma unroll
            for (int j = 0; j < NGW; ++j)
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    asm volatile("" : "+v"(acc[j][b][0]));
        }
    }

    // lane holds D[4 g + i][r16] of (row group j, token block b): outputs
    // o0 + 16 j + 4 g + i of the wave for token 16 b + r16, i.e. four
    // consecutive outputs, stored as one 8-byte write when all are in range
    // and aligned
    if (!EARLY) {
        if (r16 >= m)
            return;
        load_epilogue();
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const int mi = 16 * b + r16;
        if (mi >= m)
            continue;
#pragma unroll
        for (int j = 0; j < NO; ++j) {
            const int ob = (int)o0 + 16 * j + 4 * g;
            if (ob >= n32)
                continue;
            uint16_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if constexpr (GEGLU) {
                    const float a = __builtin_fmaf(acc[j][b][0][i], half4_at(sa[j], i), half4_at(ba[j], i));
                    const float bb = __builtin_fmaf(acc[j + NO][b][0][i], half4_at(sv[j], i), half4_at(bv[j], i));
                    v = gelu_erf(a) * bb;
                } else {
                    v = __builtin_fmaf(acc[j][b][0][i], half4_at(sa[j], i), half4_at(ba[j], i));
                }
                h[i] = output_half_bits(v);
            }
            uint16_t *dst = y + (int64_t)mi * n_out + ob;
            if (vec && ob + 3 < n32) {
                *reinterpret_cast<uint2 *>(dst) =
                    uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (ob + i < n32)
                        dst[i] = h[i];
            }
        }
    }
}

template <int KU, int RG, int W, int D, int MB, int MR, int NGW, bool EVEN, bool GEGLU, bool TILED,
          int CB, bool ZP>
void launch_decode_t(const void *x, int m, int64_t k, const void *packed, const void *scales,
                     int64_t n_out, const void *bias, const void *zeros, void *y, hipStream_t stream)
{
    constexpr int OUTW = GEGLU ? 8 * NGW : 16 * NGW;
    const unsigned grid = (unsigned)ceil_div(n_out, OUTW * RG);
    hipLaunchKernelGGL((decode_kernel<KU, RG, W, D, MB, MR, NGW, EVEN, GEGLU, TILED, CB, ZP>),
                       dim3(grid), dim3(W * kWave), 0, stream, static_cast<const uint16_t *>(x), m, k,
                       static_cast<const uint8_t *>(packed), static_cast<const uint16_t *>(scales),
                       n_out, static_cast<const uint16_t *>(bias), static_cast<const uint8_t *>(zeros),
                       static_cast<uint16_t *>(y));
}

// Reduction evenness of a launch.
template <int KU, int RG, int W, int D, int MB, int MR, int NGW, bool GEGLU, bool TILED, int CB,
          bool ZP>
void launch_decode_e(const void *x, int m, int64_t k, const void *packed, const void *scales,
                     int64_t n_out, const void *bias, const void *zeros, void *y, hipStream_t stream)
{
    if (k % (128 * KU * (W / RG)) == 0)
        launch_decode_t<KU, RG, W, D, MB, MR, NGW, true, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales,
                                                                           n_out, bias, zeros, y, stream);
    else
        launch_decode_t<KU, RG, W, D, MB, MR, NGW, false, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales,
                                                                            n_out, bias, zeros, y, stream);
}

// Launch shapes per token class and weight height (rows = n, or 2 f for
// GeGLU), from sweeps over KU, RG, W, D and NGW on MI355X at the GLM-130B
// shapes (12288, 36864 and 65536 rows; 12288 and 32768 columns) and at
// their 2-, 4- and 8-way tensor-parallel shards (4608 to 32768 rows, 1536
// to 16384 columns).  Each workgroup reads the activations once for all its
// rows, so tall matrices want many rows per workgroup, spread over more
// wavefronts (W up to 16) rather than more row groups per wavefront (which
// costs registers and occupancy); for the 36864-row QKV projection, 144 rows
// per workgroup (3 row sets x 4 K-parts, 12 wavefronts) make exactly one
// workgroup per CU.  Shorter matrices want fewer rows per workgroup, so that
// the grid still covers the 256 CUs (below about 8192 rows: 16 or 32 rows),
// and more reduction splits (more wavefronts per row); a short reduction
// (k <= 4096) wants a short round (128 or 256 columns per K-part), or the
// ring never fills; a long one (the 32768-column FFN-down at m <= 8) wants
// three row groups per wavefront and eight K-parts (36.8 against 38.7 us).
// At m <= 8 the 2-way QKV shard band (16384 to 24575 rows) takes two row
// sets of three groups (18432 x 12288 on quantized normal weights:
// 21.6-22.0 against 23.4-23.6 us).  More token blocks want more row groups
// per wavefront (each activation operand feeds more MFMAs).  At m > 48 tall
// weights keep three weight register sets in flight (D = 3): the round there
// is long enough that two sets leave the wave waiting on the loads.
template <bool GEGLU, bool TILED, bool ZP>
hipError_t launch_decode_layout4(const void *x, int m, int64_t k, const void *packed,
                                 const void *scales, int64_t n_out, const void *bias,
                                 const void *zeros, void *y, hipStream_t stream)
{
    constexpr int CB = 4;
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
#define W4_DEC(KU, RG, W, D, MB, MR, NGW)                                                      \
    launch_decode_e<KU, RG, W, D, MB, MR, NGW, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, \
                                                                     bias, zeros, y, stream)
    if constexpr (GEGLU) {
        // a wavefront always holds gate and value groups: NGW even.
        // Height bands: 3 from 49152 rows, 2 from 24576, 1 from 12288, 0 below.
        const int b = rows >= 49152 ? 3 : rows >= 24576 ? 2 : rows >= 12288 ? 1 : 0;
        if (m <= 4)
            b == 3   ? W4_DEC(2, 4, 8, 2, 1, 4, 2)
            : b == 2 ? W4_DEC(2, 2, 4, 2, 1, 4, 2)
            : b == 1 ? W4_DEC(2, 1, 4, 2, 1, 4, 2)
                     : W4_DEC(2, 1, 8, 2, 1, 4, 2);
        else if (m <= 8)
            b == 3 ? W4_DEC(2, 4, 4, 2, 1, 8, 2)
            : b    ? W4_DEC(2, 2, 8, 2, 1, 8, 2)
                   : W4_DEC(2, 1, 8, 2, 1, 8, 2);
        else if (m <= 16)
            b == 3   ? W4_DEC(2, 8, 16, 2, 1, 16, 2)
            : b == 2 ? W4_DEC(2, 4, 16, 2, 1, 16, 2)
            : b == 1 ? W4_DEC(2, 2, 8, 2, 1, 16, 2)
                     : W4_DEC(2, 1, 8, 2, 1, 16, 2);
        else if (m <= 32)
            b == 3   ? W4_DEC(1, 4, 8, 2, 2, 32, 4)
            : b == 2 ? W4_DEC(1, 2, 8, 2, 2, 32, 4)
            : b == 1 ? W4_DEC(2, 2, 8, 2, 2, 32, 2)
                     : W4_DEC(2, 1, 4, 2, 2, 32, 2);
        else if (m <= 48)
            b == 3   ? W4_DEC(1, 4, 8, 2, 3, 48, 4)
            : b == 2 ? W4_DEC(1, 4, 16, 2, 3, 48, 2)
            : b == 1 ? W4_DEC(1, 1, 4, 2, 3, 48, 4)
                     : W4_DEC(1, 1, 4, 3, 3, 48, 2);
        else
            b == 3   ? W4_DEC(1, 8, 16, 3, 4, 64, 2)
            : b == 2 ? W4_DEC(1, 4, 8, 3, 4, 64, 2)
            : b == 1 ? W4_DEC(2, 2, 4, 2, 4, 64, 2)
                     : W4_DEC(1, 1, 4, 3, 4, 64, 2);
    } else {
        // Height bands: 4 from 49152 rows, 3 from 24576, 2 from 16384,
        // 1 from 8192, 0 below.
        const int b = rows >= 49152 ? 4 : rows >= 24576 ? 3 : rows >= 16384 ? 2 : rows >= 8192 ? 1 : 0;
        if (m <= 4)
            b == 4   ? W4_DEC(2, 4, 4, 2, 1, 4, 1)
            : b == 3 ? W4_DEC(2, 3, 6, 2, 1, 4, 1)
            : b      ? W4_DEC(2, 1, 4, 2, 1, 4, 1)
                     : W4_DEC(2, 1, 8, 2, 1, 4, 1);
        else if (m <= 8)
            b == 4   ? W4_DEC(2, 4, 4, 2, 1, 8, 1)
            : b == 3 ? W4_DEC(1, 1, 4, 2, 1, 8, 3)
            : b == 2 ? W4_DEC(2, 2, 8, 2, 1, 8, 3)
            : b == 1 ? (k < 4096    ? W4_DEC(1, 1, 4, 2, 1, 8, 1)
                        : k >= 24576 ? W4_DEC(2, 1, 8, 2, 1, 8, 3)
                                     : W4_DEC(4, 3, 12, 2, 1, 8, 1))
                     : W4_DEC(2, 2, 8, 2, 1, 8, 1);
        else if (m <= 16)
            b == 4   ? W4_DEC(2, 4, 4, 2, 1, 16, 2)
            : b == 3 ? W4_DEC(2, 3, 12, 2, 1, 16, 3)
            : b == 2 ? W4_DEC(1, 3, 12, 3, 1, 16, 2)
            : b == 1 ? (k < 4096 ? W4_DEC(1, 3, 12, 2, 1, 16, 1) : W4_DEC(2, 1, 8, 2, 1, 16, 3))
                     : W4_DEC(2, 1, 8, 2, 1, 16, 2);
        else if (m <= 32)
            b == 4   ? W4_DEC(1, 2, 4, 2, 2, 32, 4)
            : b == 3 ? W4_DEC(2, 3, 12, 2, 2, 32, 3)
            : b == 2 ? W4_DEC(2, 2, 8, 2, 2, 32, 3)
            : b == 1 ? (k < 4096 ? W4_DEC(1, 3, 12, 3, 2, 32, 1)
                        : k == 4096 ? W4_DEC(1, 2, 8, 2, 2, 32, 2)
                                    : W4_DEC(2, 1, 4, 2, 2, 32, 3))
                     : W4_DEC(2, 1, 4, 2, 2, 32, 2);
        else if (m <= 48)
            b == 4   ? W4_DEC(1, 4, 8, 2, 3, 48, 4)
            : b == 3 ? W4_DEC(1, 3, 12, 2, 3, 48, 3)
            : b == 2 ? W4_DEC(1, 2, 8, 2, 3, 48, 3)
            : b == 1 ? (k < 4096 ? W4_DEC(1, 3, 12, 3, 3, 48, 1) : W4_DEC(1, 1, 4, 2, 3, 48, 3))
                     : W4_DEC(1, 1, 4, 3, 3, 48, 2);
        else
            b == 4   ? W4_DEC(1, 8, 16, 3, 4, 64, 2)
            : b == 3 ? W4_DEC(1, 3, 12, 3, 4, 64, 3)
            : b == 2 ? W4_DEC(1, 2, 8, 2, 4, 64, 3)
            : b == 1 ? (k < 4096 ? W4_DEC(1, 3, 12, 3, 4, 64, 1) : W4_DEC(1, 1, 4, 2, 4, 64, 3))
                     : W4_DEC(1, 1, 4, 3, 4, 64, 2);
    }
#undef W4_DEC
    return hipGetLastError();
}

}  // namespace w4a16
