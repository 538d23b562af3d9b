// Decode W4A16 GEMV / skinny GEMM (m <= 64) for gfx950.
//
// y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r])   (GLM-130B paper
// card, "Method": linear_forward with the weights turned back into FP16 at
// run time; paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s").
// At decode sizes the packed weights dominate the traffic (k/2 bytes per
// row against 2 m k bytes of activations), so both kernels here are built
// to stream the weights from HBM once at full bandwidth:
//
//  * Codes become exact fp16 integers in registers (dequant8: 1.25 VALU ops
//    per code) and feed v_mfma_f32_16x16x32_f16 with 16 weight rows as the
//    A operand and up to 16 tokens per MFMA as the B operand, fp32
//    accumulation.  Padding m up to 16 costs idle MFMA slots, not bytes.
//  * Every load is an unconditional range-checked buffer load (padding
//    lanes read zeros), and the main loops are unrolled twice over two
//    register sets, so the next stage's loads stay in flight while the
//    current stage is multiplied (no register copies that would force the
//    loads to retire).
//  * The row scale is constant along the sum, so it is applied once to the
//    fp32 sum in the epilogue instead of to every weight; then the bias,
//    the optional GeGLU, and one fp16 rounding.
#include "common.hpp"

namespace w4a16 {

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b)
{
    return (a + b - 1) / b;
}

// ---------------------------------------------------------------------------
// Small-batch decode (m <= 16): one 16-token MFMA block.
//
// A workgroup of 4 wavefronts owns RG groups of 16 outputs; the KS = 4 / RG
// wavefronts of a group split the reduction into interleaved chunks of
// 128 KU indices.  A wavefront streams its rows chunk by chunk (KU 16-byte
// pieces per lane per row), with a ring of D register sets so the pieces of
// the next D - 1 chunks are in flight while the current one is multiplied.
// The activation chunks of a round (KS chunks, MR x 128 KU fp16 each, MR =
// m rounded up to 4, 8 or 16) are loaded once per workgroup, permuted into
// the dequant8 operand order and double-buffered in LDS, one barrier per
// round; the RG wavefronts that work on the same chunk share it.  Each
// round's activation loads are issued before its weight loads: vector
// loads retire in order, so waiting for the activations does not wait for
// the weights.  Partial sums of the KS wavefronts of a group meet in LDS in
// a fixed order.
//
// The dequantization is the bulk of the VALU work (10 ops per 8 codes), so
// everything else is kept off the VALU: every lane's load offset is a
// per-lane constant plus a wave-uniform step.  Rows past the end are
// clamped to the last row and tokens past m to token m - 1 (they only feed
// MFMA columns and rows that are never stored); a chunk past the end gets
// the out-of-range step, so its loads return zeros.  EVEN (k a multiple of
// the 128 KU KS-index round) needs no per-lane reduction-index checks; the
// general instantiation adds them for a ragged last round.
//
// TILED selects the prepacked weight layout (w4a16_prepack): each 16-row x
// 128-index tile is one contiguous 1 KB block in lane order, so a
// wavefront reads KU KB of consecutive memory per chunk instead of 16 row
// segments of 64 KU bytes.
// ---------------------------------------------------------------------------
template <int KU, int RG, int D, int MR, bool EVEN, bool GEGLU, bool TILED>
__global__ __launch_bounds__(4 * kWave) void decode_small_kernel(
    const uint16_t *__restrict__ x, int m, int64_t k, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scales, int64_t n_out, const uint16_t *__restrict__ bias,
    uint16_t *__restrict__ y)
{
    constexpr int NG = GEGLU ? 2 : 1;
    constexpr int KS = 4 / RG;
    constexpr int KC = 128 * KU;              // reduction indices per chunk
    constexpr int LD = KC + 8;                // LDS row stride (halves): +16 bytes against bank conflicts
    constexpr int RP = KC / 8;                // 16-byte pieces per activation row per chunk
    constexpr int NPC = KS * MR * RP;                // activation pieces per round
    constexpr int XP = (NPC + 4 * kWave - 1) / (4 * kWave);   // per thread
    static_assert(NPC % (4 * kWave) == 0 || NPC < 4 * kWave, "activation pieces must divide evenly");
    static_assert(D % 2 == 0, "the LDS double buffer alternates with the round parity");
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][KS][MR][LD];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int rgi = wave % RG;
    const int kp = wave / RG;
    const int r16 = lane % 16;
    const int g = lane / 16;
    const int64_t o0 = ((int64_t)blockIdx.x * RG + rgi) * 16;   // first output of this group
    const int64_t kb = k / 2;
    const int64_t kt = ceil_div(k, 128);

    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, weight_bytes(TILED, rows, k));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (int64_t)m * k * 2);

    // Per-lane constant part of each weight load offset.  Output rows past
    // n_out: the prepacked layout holds zero rows there; the row-major one
    // is clamped to the last row (the result is never stored).
    uint32_t wbase[NG];
    {
        int64_t o = o0 + r16;
        if (!TILED && o >= n_out)
            o = n_out - 1;
        wbase[0] = TILED ? (uint32_t)((o >> 4) * kt * 1024 + 16 * lane)
                         : (uint32_t)(o * kb + 16 * g);
        if (GEGLU) {
            const int64_t ov = n_out + o;
            wbase[NG - 1] = TILED ? (uint32_t)((ov >> 4) * kt * 1024 + 16 * lane)
                                  : (uint32_t)(ov * kb + 16 * g);
        }
    }
    const uint32_t k32 = (uint32_t)k;

    // two independent accumulator chains per group (even / odd pieces)
    float4v acc[NG][2];
#pragma unroll
    for (int j = 0; j < NG; ++j)
        acc[j][0] = acc[j][1] = float4v{0.f, 0.f, 0.f, 0.f};

    const int64_t nch = ceil_div(k, KC);
    const int64_t rounds = ceil_div(nch, KS);

    // Chunk c of this wave, piece p: reduction indices c KC + 128 p + 32 g.
    // The wave-uniform step (c KC + 128 p) / 2 bytes (row-major) or tile
    // c KU + p (prepacked) is added to the per-lane base.
    auto load_w = [&](int64_t r, u32x4(&wd)[NG][KU]) {
        const uint32_t c = (uint32_t)(r * KS + kp);
        const bool live = c < (uint32_t)nch;
#pragma unroll
        for (int p = 0; p < KU; ++p) {
            const uint32_t u = c * KC + 128 * p;
            uint32_t step = TILED ? (c * KU + p) * 1024u : u / 2;
            if (!live)
                step = kOutOfRange;
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                uint32_t off = wbase[j] + step;
                if (!EVEN && !TILED && u + 32 * g >= k32)
                    off = kOutOfRange;                 // ragged last piece, row-major only
                wd[j][p] = buf_load16_stream(wrs, off);
            }
        }
    };
    // activation pieces of a round: (chunk slot, row < MR, piece) over 256 threads
    u32x4 xr[XP];
    uint32_t xbase[XP], xcol[XP];
#pragma unroll
    for (int i = 0; i < XP; ++i) {
        // threads past the last piece repeat one (same value, same LDS address)
        const int idx = (threadIdx.x + 4 * kWave * i) % NPC;
        const int q = idx / RP;                       // slot * MR + row
        const int mi = q % MR < m ? q % MR : m - 1;   // tokens past m repeat token m - 1
        xcol[i] = (uint32_t)((q / MR) * KC + 8 * (idx % RP));   // index within the round
        xbase[i] = (uint32_t)(mi * k * 2 + 2 * xcol[i]);
    }
    auto load_x = [&](int64_t r) {
        const uint32_t k0 = (uint32_t)(r * KS * KC);
        const uint32_t step = r < rounds ? 2 * k0 : kOutOfRange;
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            uint32_t off = xbase[i] + step;
            if (!EVEN && k0 + xcol[i] >= k32)
                off = kOutOfRange;
            xr[i] = buf_load16(xrs, off);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int idx = (threadIdx.x + 4 * kWave * i) % NPC;
            const int q = idx / RP;
            *reinterpret_cast<u32x4 *>(&xs[buf][q / MR][q % MR][8 * (idx % RP)]) = permute_x8(xr[i]);
        }
    };
    const int brow = r16 < MR ? r16 : MR - 1;          // MFMA columns past MR repeat row MR - 1
    auto compute = [&](int buf, const u32x4(&wd)[NG][KU]) {
        const uint16_t *xb = &xs[buf][kp][brow][32 * g];
#pragma unroll
        for (int p = 0; p < KU; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const half8 bx = as_half8(*reinterpret_cast<const u32x4 *>(xb + 128 * p + 8 * t));
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    acc[j][t & 1] = mfma16x16x32(dequant8(wd[j][p][t]), bx, acc[j][t & 1]);
            }
    };

    // Ring of D weight register sets: round r uses set r % D, loaded D - 1
    // rounds earlier.  The round loop is unrolled D times so every set has
    // a fixed register name (no copies, which would force the loads to
    // retire early).
    u32x4 wr[D][NG][KU];
    load_x(0);
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
        load_w(i, wr[i]);
    store_x(0);
    __syncthreads();
    for (int64_t r0 = 0; r0 < rounds; r0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int64_t r = r0 + i;
            if (r >= rounds)
                break;
            load_x(r + 1);
            load_w(r + D - 1, wr[(i + D - 1) % D]);
            compute(i & 1, wr[i]);
            store_x((i & 1) ^ 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int j = 0; j < NG; ++j)
        acc[j][0] += acc[j][1];

    if (KS > 1) {
        // partial sums of K-parts 1..KS-1 -> LDS; K-part 0 adds them in order
        static_assert(sizeof(xs) >= (KS - 1) * RG * NG * kWave * 4 * sizeof(float),
                      "reduction slots reuse the activation buffer");
        float *red = reinterpret_cast<float *>(&xs[0][0][0][0]);
        if (kp > 0) {
#pragma unroll
            for (int j = 0; j < NG; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[((((kp - 1) * RG + rgi) * NG + j) * kWave + lane) * 4 + i] = acc[j][0][i];
        }
        __syncthreads();
        if (kp > 0)
            return;
#pragma unroll
        for (int q = 1; q < KS; ++q)
#pragma unroll
            for (int j = 0; j < NG; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[j][0][i] += red[((((q - 1) * RG + rgi) * NG + j) * kWave + lane) * 4 + i];
    }

    // lane holds D[4 g + i][r16]: output o0 + 4 g + i, token r16
    if (r16 < m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t o = o0 + 4 * g + i;
            if (o >= n_out)
                continue;
            float v;
            if (GEGLU) {
                float a = acc[0][0][i] * half_bits_to_float(scales[o]);
                float bv = acc[NG - 1][0][i] * half_bits_to_float(scales[n_out + o]);
                if (bias) {
                    a += half_bits_to_float(bias[o]);
                    bv += half_bits_to_float(bias[n_out + o]);
                }
                v = gelu_erf(a) * bv;
            } else {
                v = acc[0][0][i] * half_bits_to_float(scales[o]);
                if (bias)
                    v += half_bits_to_float(bias[o]);
            }
            y[(int64_t)r16 * n_out + o] = float_to_half_bits(v);
        }
    }
}

template <int KU, int RG, int D, int MR, bool EVEN, bool GEGLU, bool TILED>
void launch_decode_small_t(const void *x, int m, int64_t k, const void *packed, const void *scales,
                           int64_t n_out, const void *bias, void *y, hipStream_t stream)
{
    const unsigned grid = (unsigned)ceil_div(n_out, 16 * RG);
    hipLaunchKernelGGL((decode_small_kernel<KU, RG, D, MR, EVEN, GEGLU, TILED>), dim3(grid),
                       dim3(4 * kWave), 0, stream, static_cast<const uint16_t *>(x), m, k,
                       static_cast<const uint8_t *>(packed), static_cast<const uint16_t *>(scales),
                       n_out, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
}

// Token-count class and reduction evenness of a small-batch launch.
template <int KU, int RG, int D, bool GEGLU, bool TILED>
void launch_decode_small(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, void *y, hipStream_t stream)
{
    const bool even = k % (128 * KU * (4 / RG)) == 0;
#define W4_SMALL(MR, EV)                                                                          \
    launch_decode_small_t<KU, RG, D, MR, EV, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, \
                                                           stream)
    if (m <= 4) {
        if (even) W4_SMALL(4, true); else W4_SMALL(4, false);
    } else if (m <= 8) {
        if (even) W4_SMALL(8, true); else W4_SMALL(8, false);
    } else {
        if (even) W4_SMALL(16, true); else W4_SMALL(16, false);
    }
#undef W4_SMALL
}

// ---------------------------------------------------------------------------
// Mid-batch decode (16 < m <= 64): MB 16-token blocks per MFMA row group.
//
// A workgroup owns 16 NG weight rows; its W wavefronts split the reduction
// into 128 KU-wide steps taken round-robin, so the waves of a workgroup
// sweep each row front to back together.  Per step a lane loads KU
// 16-byte pieces of each of its NG rows and the matching 4 KU x 16 bytes of
// its activation row; the next step's loads are in flight while the
// current step runs.  The W partial sums meet in LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int MB, int NG, int W, int KU, bool GEGLU, bool TILED>
__global__ __launch_bounds__(W * kWave) void decode_kernel(const uint16_t *__restrict__ x, int m,
                                                          int64_t k,
                                                          const uint8_t *__restrict__ packed,
                                                          const uint16_t *__restrict__ scales,
                                                          int64_t n_out,
                                                          const uint16_t *__restrict__ bias,
                                                          uint16_t *__restrict__ y)
{
    static_assert(!GEGLU || (NG % 2 == 0), "GeGLU tiles pair gate and value groups");
    constexpr int kRowsPerWG = 16 * NG;
    constexpr int kOutPerWG = GEGLU ? kRowsPerWG / 2 : kRowsPerWG;
    constexpr int kStep = 128 * KU;          // reduction indices per wave step
    constexpr int kRed = W / 2;              // partial-sum slots (two waves per slot)
    __shared__ float red[kRed][NG][MB][kWave][4];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int r16 = lane % 16;
    const int g = lane / 16;
    const int64_t out0 = (int64_t)blockIdx.x * kOutPerWG;
    const int64_t kb = k / 2;
    const int64_t kt = ceil_div(k, 128);

    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, weight_bytes(TILED, rows, k));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (int64_t)m * k * 2);

    // base offset of the weight row held by this lane for group j
    uint32_t wbase[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        int64_t r;
        bool ok;
        if (GEGLU) {
            const int jj = j % (NG / 2);
            const int64_t f = out0 + 16 * jj + r16;
            ok = f < n_out;
            r = (j < NG / 2) ? f : n_out + f;
        } else {
            r = out0 + 16 * j + r16;
            ok = r < n_out;
        }
        wbase[j] = row_base_off<TILED>(ok ? r : -1, kb, kt, lane);
    }
    uint32_t xbase[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const int mi = 16 * b + r16;
        xbase[b] = mi < m ? (uint32_t)(mi * k * 2) : kOutOfRange;
    }
    const uint32_t k32 = (uint32_t)k;

    float4v acc[NG][MB];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = float4v{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = ceil_div(k, kStep);

    // Piece p of a step: bytes [64 p + 16 g, +16) of the row's 64 KU-byte
    // chunk, i.e. reduction indices [128 p + 32 g, +32).
    auto load_step = [&](int64_t s, u32x4(&wd)[NG][KU], u32x4(&xd)[MB][KU][4]) {
#pragma unroll
        for (int p = 0; p < KU; ++p) {
            const uint32_t kc = (uint32_t)s * kStep + 128 * p + 32 * g;
            const bool kin = kc < k32;
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    xd[b][p][t] = buf_load16(xrs, kin ? xbase[b] + 2 * (kc + 8 * t) : kOutOfRange);
            const uint32_t step = piece_step_off<TILED>(kc);
#pragma unroll
            for (int j = 0; j < NG; ++j)
                wd[j][p] = buf_load16_stream(wrs, kin ? wbase[j] + step : kOutOfRange);
        }
    };
    auto compute = [&](const u32x4(&wd)[NG][KU], const u32x4(&xd)[MB][KU][4]) {
#pragma unroll
        for (int p = 0; p < KU; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                half8 bx[MB];
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    bx[b] = as_half8(permute_x8(xd[b][p][t]));
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    const half8 a = dequant8(wd[j][p][t]);
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        acc[j][b] = mfma16x16x32(a, bx[b], acc[j][b]);
                }
            }
    };

    u32x4 wa[NG][KU], xa[MB][KU][4], wb[NG][KU], xb[MB][KU][4];
    int64_t s = wave;
    load_step(s, wa, xa);
    while (s < nsteps) {
        load_step(s + W, wb, xb);
        compute(wa, xa);
        s += W;
        if (s >= nsteps)
            break;
        load_step(s + W, wa, xa);
        compute(wb, xb);
        s += W;
    }

    // Partial sums of the W waves meet in LDS in a fixed order: the upper
    // half of the waves stores, the lower half adds its own sum on top, and
    // the epilogue adds the W / 2 slots.
    if (wave >= kRed) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[wave - kRed][j][b][lane][i] = acc[j][b][i];
    }
    __syncthreads();
    if (wave < kRed) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[wave][j][b][lane][i] = acc[j][b][i] + red[wave][j][b][lane][i];
    }
    __syncthreads();

    // D[4 (l / 16) + i][l % 16]: weight row 4 (l / 16) + i of the group, token l % 16
    auto partial = [&](int j, int rr, int mi) {
        const int b = mi / 16;
        const int l = 16 * (rr / 4) + (mi % 16);
        const int i = rr % 4;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kRed; ++w)
            v += red[w][j][b][l][i];
        return v;
    };

    const int total = kOutPerWG * m;
    for (int idx = threadIdx.x; idx < total; idx += W * kWave) {
        const int col = idx % kOutPerWG;
        const int mi = idx / kOutPerWG;
        const int64_t o = out0 + col;
        if (o >= n_out)
            continue;
        const int j = col / 16;
        const int rr = col % 16;
        float val;
        if (GEGLU) {
            float a = partial(j, rr, mi) * half_bits_to_float(scales[o]);
            float bv = partial(j + NG / 2, rr, mi) * half_bits_to_float(scales[n_out + o]);
            if (bias) {
                a += half_bits_to_float(bias[o]);
                bv += half_bits_to_float(bias[n_out + o]);
            }
            val = gelu_erf(a) * bv;
        } else {
            val = partial(j, rr, mi) * half_bits_to_float(scales[o]);
            if (bias)
                val += half_bits_to_float(bias[o]);
        }
        y[(int64_t)mi * n_out + o] = float_to_half_bits(val);
    }
}

template <int MB, int NG, int W, int KU, bool GEGLU, bool TILED>
void launch_decode_t(const void *x, int m, int64_t k, const void *packed, const void *scales,
                     int64_t n_out, const void *bias, void *y, hipStream_t stream)
{
    constexpr int out_per = GEGLU ? 8 * NG : 16 * NG;
    const unsigned grid = (unsigned)ceil_div(n_out, out_per);
    hipLaunchKernelGGL((decode_kernel<MB, NG, W, KU, GEGLU, TILED>), dim3(grid), dim3(W * kWave), 0,
                       stream, static_cast<const uint16_t *>(x), m, k,
                       static_cast<const uint8_t *>(packed), static_cast<const uint16_t *>(scales),
                       n_out, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
}

template <int MB, bool GEGLU, bool TILED>
static void launch_decode_mb(const void *x, int m, int64_t k, const void *packed,
                             const void *scales, int64_t n_out, const void *bias, void *y,
                             hipStream_t stream)
{
    // Enough workgroups to cover all 256 compute units several times over,
    // with as many rows per workgroup as that allows (fewer activation
    // re-reads per weight byte).
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    if (rows / 64 >= 512)
        launch_decode_t<MB, 4, 4, 1, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
    else
        launch_decode_t<MB, 2, 4, 1, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
}

template <bool TILED>
static hipError_t launch_decode_layout(const void *x, int m, int64_t k, const void *packed,
                                       const void *scales, int64_t n_out, const void *bias, void *y,
                                       bool geglu, hipStream_t stream)
{
    if (m <= 16) {
        if (geglu)
            launch_decode_small<2, 2, 2, true, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
        else
            launch_decode_small<2, 2, 2, false, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
        return hipGetLastError();
    }
    const int mb = (m + 15) / 16;
#define W4_DECODE_CASE(MBV)                                                                       \
    case MBV:                                                                                     \
        if (geglu)                                                                                \
            launch_decode_mb<MBV, true, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);  \
        else                                                                                      \
            launch_decode_mb<MBV, false, TILED>(x, m, k, packed, scales, n_out, bias, y, stream); \
        break;
    switch (mb) {
        W4_DECODE_CASE(2)
        W4_DECODE_CASE(3)
        W4_DECODE_CASE(4)
    default:
        return hipErrorInvalidValue;
    }
#undef W4_DECODE_CASE
    return hipGetLastError();
}

hipError_t launch_decode(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, void *y, bool geglu, bool tiled,
                         hipStream_t stream)
{
    if (tiled)
        return launch_decode_layout<true>(x, m, k, packed, scales, n_out, bias, y, geglu, stream);
    return launch_decode_layout<false>(x, m, k, packed, scales, n_out, bias, y, geglu, stream);
}

}  // namespace w4a16
