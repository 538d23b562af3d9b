// Prefill W4A16 GEMM (m > 64) for gfx950: a compute-bound tile GEMM on the
// fp16 matrix cores with the INT4 weights dequantized on the fly.
//
// Same result definition as the decode kernel (GLM-130B paper card,
// "Method"; paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s"):
// y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r]), fp32 accumulation,
// optional fused GeGLU (paper card "Hyperparameters"; paperlayer.ai B.3).
//
// Tiling.  A 256-thread workgroup computes a 128 (weight rows) x 128
// (tokens) output tile over 128-wide reduction steps; wave w owns the
// 64 x 64 quadrant (w & 1, w >> 1), i.e. 4 x 4 MFMA 16x16 tiles.
//  * Activations: the 128 x 128 fp16 step tile is copied global -> LDS once
//    per workgroup (permuted into the operand order of dequant8 as it is
//    written), double-buffered so the next step's copy overlaps this step's
//    MFMAs.  Rows are padded to 272 bytes so the 16 lanes that read one
//    operand column hit distinct LDS banks.
//  * Weights: each lane loads its 16 packed bytes per row group straight
//    into registers (one dwordx4, prefetched a step ahead) and dequantizes
//    them into the MFMA A operand: the fp16 weight tile never exists in
//    memory.  The scale is applied once per output in the epilogue.
//  * All loads are unconditional range-checked buffer loads and the step
//    loop is unrolled twice over two weight register sets, so the next
//    step's loads stay in flight while this step's MFMAs run.
#include "common.hpp"

namespace w4a16 {

constexpr int kPBN = 128;           // weight rows per tile
constexpr int kPBM = 128;           // tokens per tile
constexpr int kPBK = 128;           // reduction step
constexpr int kPLd = kPBK + 8;      // LDS row stride in halves (272 bytes)
constexpr int kPThreads = 256;

template <bool GEGLU, bool TILED>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(const uint16_t *__restrict__ x,
                                                            int64_t m, int64_t k,
                                                            const uint8_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scales,
                                                            int64_t n_out,
                                                            const uint16_t *__restrict__ bias,
                                                            uint16_t *__restrict__ y,
                                                            int tiles_m)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][kPBM * kPLd];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int wn = wave & 1, wm = wave >> 1;
    const int r16 = lane % 16;
    const int g = lane / 16;

    const int tile_m = blockIdx.x % tiles_m;
    const int64_t tile_n = blockIdx.x / tiles_m;
    const int64_t m0 = (int64_t)tile_m * kPBM;
    constexpr int kOutPerTile = GEGLU ? kPBN / 2 : kPBN;
    const int64_t o0 = tile_n * kOutPerTile;
    const int64_t kb = k / 2;
    const int64_t kt = (k + 127) / 128;   // tiles per row group (prepacked layout)

    // base offset of the weight row of this lane in group j (4 groups of 16 per wave)
    uint32_t wbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int64_t r;
        bool ok;
        if (GEGLU) {
            const int64_t f = o0 + 32 * wn + 16 * (j % 2) + r16;
            ok = f < n_out;
            r = (j < 2) ? f : n_out + f;
        } else {
            r = o0 + 64 * wn + 16 * j + r16;
            ok = r < n_out;
        }
        wbase[j] = row_base_off<TILED>(ok ? r : -1, kb, kt, lane);
    }
    const uint32_t k32 = (uint32_t)k;

    float4v acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            acc[j][b] = float4v{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = (k + kPBK - 1) / kPBK;
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, weight_bytes(TILED, rows, k));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, m * k * 2);

    // activation copy: 128 rows x 16 pieces of 16 bytes; thread handles 8
    // pieces.  Issued before the same stage's weight loads: loads retire in
    // order, so storing them to LDS does not wait for the weights.
    u32x4 xr[8];
    uint32_t xrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + kPThreads * i;
        const int64_t mi = m0 + c / 16;
        xrow[i] = mi < m ? (uint32_t)((mi * k + 8 * (c % 16)) * 2) : kOutOfRange;
    }
    auto load_x = [&](int64_t s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = threadIdx.x + kPThreads * i;
            const uint32_t kk = (uint32_t)s * kPBK + 8 * (c % 16);
            xr[i] = buf_load16(xrs, kk < k32 ? xrow[i] + 2 * (uint32_t)s * kPBK : kOutOfRange);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = threadIdx.x + kPThreads * i;
            const int rr = c / 16;
            *reinterpret_cast<u32x4 *>(&xs[buf][rr * kPLd + 8 * (c % 16)]) = permute_x8(xr[i]);
        }
    };
    auto load_w = [&](int64_t s, u32x4(&wd)[4]) {
        const uint32_t kc = (uint32_t)s * kPBK + 32 * g;
        const uint32_t step = piece_step_off<TILED>(kc);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wd[j] = buf_load16_stream(wrs, kc < k32 ? wbase[j] + step : kOutOfRange);
    };
    auto compute = [&](int buf, const u32x4(&wd)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 bx[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int rr = 64 * wm + 16 * b + r16;
                bx[b] = as_half8(*reinterpret_cast<const u32x4 *>(&xs[buf][rr * kPLd + 32 * g + 8 * t]));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const half8 a = dequant8(wd[j][t]);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[j][b] = mfma16x16x32(a, bx[b], acc[j][b]);
            }
        }
    };

    // two register sets for the weights, used alternately (the loop is
    // unrolled twice so no set is ever copied)
    u32x4 wa[4], wb[4];
    load_x(0);
    load_w(0, wa);
    store_x(0);
    __syncthreads();
    for (int64_t s = 0;;) {
        load_x(s + 1);
        load_w(s + 1, wb);
        compute(0, wa);
        store_x(1);
        __syncthreads();
        if (++s >= nsteps)
            break;
        load_x(s + 1);
        load_w(s + 1, wa);
        compute(1, wb);
        store_x(0);
        __syncthreads();
        if (++s >= nsteps)
            break;
    }

    // epilogue: lane holds D[4 g + i][r16] of tile (j, b): weight row 4 g + i, token r16
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t mi = m0 + 64 * wm + 16 * b + r16;
        if (mi >= m)
            continue;
        if (GEGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t f = o0 + 32 * wn + 16 * j + 4 * g + i;
                    if (f >= n_out)
                        continue;
                    float a = acc[j][b][i] * half_bits_to_float(scales[f]);
                    float bv = acc[j + 2][b][i] * half_bits_to_float(scales[n_out + f]);
                    if (bias) {
                        a += half_bits_to_float(bias[f]);
                        bv += half_bits_to_float(bias[n_out + f]);
                    }
                    y[mi * n_out + f] = float_to_half_bits(gelu_erf(a) * bv);
                }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t n = o0 + 64 * wn + 16 * j + 4 * g + i;
                    if (n >= n_out)
                        continue;
                    float v = acc[j][b][i] * half_bits_to_float(scales[n]);
                    if (bias)
                        v += half_bits_to_float(bias[n]);
                    y[mi * n_out + n] = float_to_half_bits(v);
                }
        }
    }
}

hipError_t launch_prefill(const void *x, int64_t m, int64_t k, const void *packed,
                          const void *scales, int64_t n_out, const void *bias, void *y, bool geglu,
                          bool tiled, hipStream_t stream)
{
    const int64_t out_per = geglu ? kPBN / 2 : kPBN;
    const int64_t tiles_n = (n_out + out_per - 1) / out_per;
    const int64_t tiles_m = (m + kPBM - 1) / kPBM;
    const int64_t grid = tiles_n * tiles_m;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const uint8_t *pp = static_cast<const uint8_t *>(packed);
    const uint16_t *sp = static_cast<const uint16_t *>(scales);
    const uint16_t *bp = static_cast<const uint16_t *>(bias);
    uint16_t *yp = static_cast<uint16_t *>(y);
#define W4_PREFILL(G, T)                                                                          \
    hipLaunchKernelGGL((prefill_kernel<G, T>), dim3((unsigned)grid), dim3(kPThreads), 0, stream, xp, \
                       m, k, pp, sp, n_out, bp, yp, (int)tiles_m)
    if (geglu && tiled)
        W4_PREFILL(true, true);
    else if (geglu)
        W4_PREFILL(true, false);
    else if (tiled)
        W4_PREFILL(false, true);
    else
        W4_PREFILL(false, false);
#undef W4_PREFILL
    return hipGetLastError();
}

}  // namespace w4a16
