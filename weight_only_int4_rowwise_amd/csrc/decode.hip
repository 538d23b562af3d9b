// Decode W4A16 GEMV / skinny GEMM (m <= 64) for gfx950.
//
// y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r])   (GLM-130B paper
// card, "Method": linear_forward with the weights turned back into FP16 at
// run time; paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s").
// At decode sizes the packed weights dominate the traffic (k/2 bytes per
// row against 2 m k bytes of activations), so the kernel is built to stream
// them from HBM once at full bandwidth:
//
//  * A workgroup owns 16 * NG weight rows; its W wavefronts split the
//    reduction dimension into 128-wide steps taken round-robin, so the
//    waves of one workgroup sweep each row front to back together.
//  * Per step a lane loads 16 contiguous bytes (32 codes) of each of its NG
//    rows with one non-temporal dwordx4, and 4 x 16 bytes of its activation
//    row; the next step's loads are in flight while the current step runs.
//  * Codes become exact fp16 integers in registers (dequant8: 1.25 VALU ops
//    per code) and feed v_mfma_f32_16x16x32_f16 with the weights as the
//    16-row A operand and up to 16 tokens per MFMA as the B operand, fp32
//    accumulation.  Padding m up to 16 costs idle MFMA slots, not bytes.
//  * The W partial sums meet in LDS in a fixed order (deterministic), and
//    the epilogue applies the row scale (constant along the sum, so it is
//    applied once to the fp32 sum instead of to every weight), the bias,
//    the optional GeGLU, and one fp16 rounding.
#include "common.hpp"

namespace w4a16 {

template <int MB, int NG, int W, bool GEGLU>
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
    __shared__ float red[W][NG][MB][kWave][4];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int r16 = lane % 16;
    const int g = lane / 16;
    const int64_t out0 = (int64_t)blockIdx.x * kOutPerWG;
    const int64_t kb = k / 2;   // bytes per packed row

    // weight row held by this lane for group j, or -1 past the end
    int64_t row[NG];
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
        row[j] = ok ? r : -1;
    }

    float4v acc[NG][MB];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[j][b] = float4v{0.f, 0.f, 0.f, 0.f};

    const int64_t nsteps = (k + 127) / 128;

    u32x4 wv[NG], xv[MB][4];
    auto load_step = [&](int64_t s, u32x4(&wd)[NG], u32x4(&xd)[MB][4]) {
        const int64_t kc = s * 128 + 32 * g;   // first reduction index of this lane's chunk
        const bool kin = (s < nsteps) && (kc < k);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (kin && row[j] >= 0)
                wd[j] = load_stream16(packed + row[j] * kb + kc / 2);
            else
                wd[j] = u32x4{0u, 0u, 0u, 0u};   // code 0
        }
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const int mi = 16 * b + r16;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (kin && mi < m)
                    xd[b][t] = load16(x + (int64_t)mi * k + kc + 8 * t);
                else
                    xd[b][t] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    int64_t s = wave;
    load_step(s, wv, xv);
    for (; s < nsteps; s += W) {
        u32x4 wn[NG], xn[MB][4];
        load_step(s + W, wn, xn);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 bx[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b)
                bx[b] = as_half8(permute_x8(xv[b][t]));
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                const half8 a = dequant8(wv[j][t]);
#pragma unroll
                for (int b = 0; b < MB; ++b)
                    acc[j][b] = mfma16x16x32(a, bx[b], acc[j][b]);
            }
        }
#pragma unroll
        for (int j = 0; j < NG; ++j)
            wv[j] = wn[j];
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xv[b][t] = xn[b][t];
    }

    // partial sums of the W waves -> LDS, fixed summation order below
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[wave][j][b][lane][i] = acc[j][b][i];
    __syncthreads();

    // D[4 (l / 16) + i][l % 16]: weight row 4 (l / 16) + i of the group, token l % 16
    auto partial = [&](int j, int rr, int mi) {
        const int b = mi / 16;
        const int l = 16 * (rr / 4) + (mi % 16);
        const int i = rr % 4;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w)
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

template <int MB, int NG, bool GEGLU>
static void launch_decode_t(const void *x, int m, int64_t k, const void *packed, const void *scales,
                            int64_t n_out, const void *bias, void *y, hipStream_t stream)
{
    constexpr int W = 4;
    constexpr int out_per = GEGLU ? 8 * NG : 16 * NG;
    const unsigned grid = (unsigned)((n_out + out_per - 1) / out_per);
    hipLaunchKernelGGL((decode_kernel<MB, NG, W, GEGLU>), dim3(grid), dim3(W * kWave), 0, stream,
                       static_cast<const uint16_t *>(x), m, k, static_cast<const uint8_t *>(packed),
                       static_cast<const uint16_t *>(scales), n_out,
                       static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
}

template <int MB, bool GEGLU>
static void launch_decode_mb(const void *x, int m, int64_t k, const void *packed,
                             const void *scales, int64_t n_out, const void *bias, void *y,
                             hipStream_t stream)
{
    // Enough workgroups to cover all 256 compute units several times over,
    // with as many rows per workgroup as that allows (fewer activation
    // re-reads per weight byte).
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    if (rows / 64 >= 512)
        launch_decode_t<MB, 4, GEGLU>(x, m, k, packed, scales, n_out, bias, y, stream);
    else
        launch_decode_t<MB, 2, GEGLU>(x, m, k, packed, scales, n_out, bias, y, stream);
}

hipError_t launch_decode(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, void *y, bool geglu, hipStream_t stream)
{
    const int mb = (m + 15) / 16;
#define W4_DECODE_CASE(MBV)                                                                       \
    case MBV:                                                                                     \
        if (geglu)                                                                                \
            launch_decode_mb<MBV, true>(x, m, k, packed, scales, n_out, bias, y, stream);         \
        else                                                                                      \
            launch_decode_mb<MBV, false>(x, m, k, packed, scales, n_out, bias, y, stream);        \
        break;
    switch (mb) {
        W4_DECODE_CASE(1)
        W4_DECODE_CASE(2)
        W4_DECODE_CASE(3)
        W4_DECODE_CASE(4)
    default:
        return hipErrorInvalidValue;
    }
#undef W4_DECODE_CASE
    return hipGetLastError();
}

}  // namespace w4a16
