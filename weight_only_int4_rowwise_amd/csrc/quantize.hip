// Row-parallel absmax INT4 quantizer for gfx950 (the one-off weight
// compression step of GLM-130B's weight-only INT4 scheme).
//
// Per output row r of W fp16 [n][k]  (GLM-130B paper card, "Method"
// pseudocode and "Paper vs code", bullet "Quantization scale"):
//   a    = max_c |W[r][c]|
//   s    = fp16(a / 7)                     stored scale (divisor 2^(b-1)-1)
//   q[c] = clamp(round_half_even(W[r][c] / s), -7, 7),  0 if s == 0
//   packed two codes per byte (layout in include/w4a16.h).
//
// One 256-thread workgroup owns one row.  Each thread loads its 16-byte
// chunks of the row once (coalesced), keeps them in registers, and the
// absmax is reduced across the wavefront with cross-lane shuffles and across
// the four wavefronts through LDS.  The codes are formed from the registers,
// so HBM is read once and written once (2k + k/2 + 2 bytes per row).
//
// Exactness.  |w| as a bit pattern (sign cleared) orders like its value for
// finite inputs, so the absmax is an integer max.  a / 7 is a correctly
// rounded fp32 division, and fp32 -> fp16 rounding after it gives the
// correctly rounded fp16 quotient (24 >= 2 * 11 + 2 bits, so the double
// rounding is harmless).  For the codes, r = |w| * (1/s) is within 2^-20 of
// the exact quotient |w| / s (for quotients <= 16); a quotient of two fp16
// numbers that is not a half-integer lies at least 2^-12 from every
// half-integer, so rounding r gives the exact result, and |r - (j + 1/2)| <
// 2^-13 identifies an exact tie, which goes to the even neighbour.
#include "common.hpp"

namespace w4a16 {

constexpr int kQThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
    return v;
}

// Row absmax bit pattern (sign cleared) over the workgroup.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *lds4)
{
    v = wave_max_u32(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0)
        lds4[wave] = v;
    __syncthreads();
    uint32_t r = max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]));
    return r;
}

struct RowScale {
    float s;      // scale as fp32 (exact copy of the fp16 value)
    float inv;    // 1 / s (fp32, correctly rounded); unused when s == 0
    uint16_t bits;
};

__device__ __forceinline__ RowScale make_scale(uint32_t amax_bits)
{
    const float a = half_bits_to_float((uint16_t)amax_bits);
    const uint16_t sb = float_to_half_bits(__fdiv_rn(a, 7.0f));
    RowScale rs;
    rs.bits = sb;
    rs.s = half_bits_to_float(sb);
    rs.inv = rs.s != 0.0f ? __fdiv_rn(1.0f, rs.s) : 0.0f;
    return rs;
}

// Code of one fp16 weight (bit pattern) as a 4-bit two's-complement nibble.
__device__ __forceinline__ uint32_t code_nibble(uint32_t wbits, const RowScale &rs)
{
    const float mag = half_bits_to_float((uint16_t)(wbits & 0x7FFFu));
    const float r = mag * rs.inv;
    const float fl = floorf(r);
    const float d = r - fl - 0.5f;
    // exact tie -> even neighbour; otherwise nearest
    float c = fabsf(d) < 0x1p-13f ? fl + (float)((int)fl & 1) : rintf(r);
    c = fminf(c, 7.0f);
    int q = (int)c;
    if (rs.s == 0.0f)
        q = 0;
    if (wbits & 0x8000u)
        q = -q;
    return (uint32_t)q & 0xFu;
}

// Register-resident path: the row fits in kQThreads * 8 * CHUNKS halves.
// Requires k % 8 == 0 (16-byte chunks) and 16-byte aligned row starts.
template <int CHUNKS>
__global__ __launch_bounds__(kQThreads) void quantize_rows_reg(const uint16_t *__restrict__ w,
                                                               int64_t k,
                                                               uint8_t *__restrict__ packed,
                                                               uint16_t *__restrict__ scales)
{
    __shared__ uint32_t lds4[4];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * k;
    uint8_t *pr = packed + row * (k / 2);
    const int64_t nchunk = k / 8;

    u32x4 v[CHUNKS];
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int64_t idx = (int64_t)c * kQThreads + threadIdx.x;
        if (idx < nchunk) {
            v[c] = load_stream16(reinterpret_cast<const uint8_t *>(wr + idx * 8));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m = max(m, v[c][j] & 0x7FFFu);
                m = max(m, (v[c][j] >> 16) & 0x7FFFu);
            }
        }
    }
    const uint32_t amax = block_max_u32(m, lds4);
    const RowScale rs = make_scale(amax);
    if (threadIdx.x == 0)
        scales[row] = rs.bits;

#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int64_t idx = (int64_t)c * kQThreads + threadIdx.x;
        if (idx < nchunk) {
            uint32_t out = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out |= code_nibble(v[c][j] & 0xFFFFu, rs) << (8 * j);
                out |= code_nibble(v[c][j] >> 16, rs) << (8 * j + 4);
            }
            *reinterpret_cast<uint32_t *>(pr + idx * 4) = out;
        }
    }
}

// General path (any even k, any row length): two sweeps over the row; the
// second one mostly hits in cache.
__global__ __launch_bounds__(kQThreads) void quantize_rows_generic(const uint16_t *__restrict__ w,
                                                                   int64_t k,
                                                                   uint8_t *__restrict__ packed,
                                                                   uint16_t *__restrict__ scales)
{
    __shared__ uint32_t lds4[4];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * k;
    uint8_t *pr = packed + row * (k / 2);
    const int64_t npair = k / 2;
    const uint32_t *wr2 = reinterpret_cast<const uint32_t *>(wr);   // k even: 4-byte pairs

    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < npair; i += kQThreads) {
        const uint32_t p = wr2[i];
        m = max(m, p & 0x7FFFu);
        m = max(m, (p >> 16) & 0x7FFFu);
    }
    const uint32_t amax = block_max_u32(m, lds4);
    const RowScale rs = make_scale(amax);
    if (threadIdx.x == 0)
        scales[row] = rs.bits;
    for (int64_t i = threadIdx.x; i < npair; i += kQThreads) {
        const uint32_t p = wr2[i];
        pr[i] = (uint8_t)(code_nibble(p & 0xFFFFu, rs) | (code_nibble(p >> 16, rs) << 4));
    }
}

hipError_t launch_quantize(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                           hipStream_t stream)
{
    const uint16_t *wp = static_cast<const uint16_t *>(w);
    uint8_t *pp = static_cast<uint8_t *>(packed);
    uint16_t *sp = static_cast<uint16_t *>(scales);
    const dim3 grid((unsigned)n), block(kQThreads);
    if (k % 8 == 0) {
        const int64_t chunks = (k / 8 + kQThreads - 1) / kQThreads;
        if (chunks <= 1)
            hipLaunchKernelGGL(quantize_rows_reg<1>, grid, block, 0, stream, wp, k, pp, sp);
        else if (chunks <= 2)
            hipLaunchKernelGGL(quantize_rows_reg<2>, grid, block, 0, stream, wp, k, pp, sp);
        else if (chunks <= 4)
            hipLaunchKernelGGL(quantize_rows_reg<4>, grid, block, 0, stream, wp, k, pp, sp);
        else if (chunks <= 8)
            hipLaunchKernelGGL(quantize_rows_reg<8>, grid, block, 0, stream, wp, k, pp, sp);
        else if (chunks <= 16)
            hipLaunchKernelGGL(quantize_rows_reg<16>, grid, block, 0, stream, wp, k, pp, sp);
        else
            hipLaunchKernelGGL(quantize_rows_generic, grid, block, 0, stream, wp, k, pp, sp);
    } else {
        hipLaunchKernelGGL(quantize_rows_generic, grid, block, 0, stream, wp, k, pp, sp);
    }
    return hipGetLastError();
}

}  // namespace w4a16
