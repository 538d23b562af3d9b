// Row-parallel absmax INT4 quantizer for gfx950 (the one-off weight
// compression step of GLM-130B's weight-only INT4 scheme), and its INT8
// variant (divisor 127, codes in [-127, 127], one two's-complement byte per
// code: the pages' b-bit scale with b = 8).
//
// Per output row r of W fp16 [n][k]  (GLM-130B paper card, "Method"
// pseudocode and "Paper vs code", bullet "Quantization scale"):
//   a    = max_c |W[r][c]|
//   s    = fp16(a / 7)                     stored scale (divisor 2^(b-1)-1)
//   q[c] = clamp(round_half_even(W[r][c] / s), -7, 7),  0 if s == 0
//   packed two codes per byte (layout in include/w4a16.h).
//
// Rows are spread over one, two or four wavefronts (by row length).  Each
// lane loads its 16-byte chunks of the row once (coalesced, unconditional
// range-checked loads, several rows in flight per compute unit) and keeps
// them in registers; the absmax is reduced across the wavefront with
// cross-lane shuffles and across the row's wavefronts through LDS.  The
// codes are formed from the registers, so HBM is read once and written
// once (2k + k/2 + 2 bytes per row).
//
// Exactness.  |w| as a bit pattern (sign cleared) orders like its value for
// finite inputs, so the absmax is an integer max.  a / 7 is a correctly
// rounded fp32 division, and fp32 -> fp16 rounding after it gives the
// correctly rounded fp16 quotient (24 >= 2 * 11 + 2 bits, so the double
// rounding is harmless).  For the codes, r = w * (1/s) is within 2^-20 of
// the exact quotient Q = w / s (|Q| <= 10.5).  A quotient of two fp16
// numbers that is not a half-integer lies at least 2^-12 from every
// half-integer, while an exact tie is a multiple of 2^-12.  So rounding r
// to the nearest multiple of 2^-12 returns Q itself for a tie and stays on
// Q's side of every half-integer otherwise, and rounding that to an
// integer, ties to even, gives round_half_even(Q).  The gap holds for any
// |Q| (the two sides differ by an integer multiple of the significand
// spacing), so the INT8 codes follow the same steps: there |Q| < 191
// (subnormal scales included), r is within 2^-15 of Q, and adding
// 2^23 + 256 leaves q + 256 in the low mantissa bits, whose low byte is
// q's two's complement.
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

template <int QMAX>
__device__ __forceinline__ RowScale make_scale(uint32_t amax_bits)
{
    const float a = half_bits_to_float((uint16_t)amax_bits);
    const uint16_t sb = float_to_half_bits(__fdiv_rn(a, (float)QMAX));
    RowScale rs;
    rs.bits = sb;
    rs.s = half_bits_to_float(sb);
    rs.inv = rs.s != 0.0f ? __fdiv_rn(1.0f, rs.s) : 0.0f;
    return rs;
}

// Two's-complement nibble of the code of one weight (fp32 value wf), in 8
// VALU ops: r = wf / s; snap r to the 2^-12 grid ((r + 3072) - 3072 rounds
// to a multiple of 2^-12 for |r| < 1024); clamp to [-7, 7] (v_med3); adding
// 2^23 + 16 rounds to an integer, ties to even, and leaves (q + 16) in the
// low mantissa bits, whose low nibble is q mod 16.  s == 0 has inv == 0 and
// gives code 0.
__device__ __forceinline__ uint32_t code_nibble_f(float wf, float inv)
{
    const float r = wf * inv;
    const float snap = __fsub_rn(__fadd_rn(r, 3072.0f), 3072.0f);
    const float c = __builtin_amdgcn_fmed3f(snap, -7.0f, 7.0f);
    return __builtin_bit_cast(uint32_t, __fadd_rn(c, 8388624.0f)) & 0xFu;
}

// Two's-complement byte of the INT8 code of one weight: the same steps
// with the clamp at 127 and 2^23 + 256 as the rounding constant.
__device__ __forceinline__ uint32_t code_byte_f(float wf, float inv)
{
    const float r = wf * inv;
    const float snap = __fsub_rn(__fadd_rn(r, 3072.0f), 3072.0f);
    const float c = __builtin_amdgcn_fmed3f(snap, -127.0f, 127.0f);
    return __builtin_bit_cast(uint32_t, __fadd_rn(c, 8388864.0f)) & 0xFFu;
}

__device__ __forceinline__ uint32_t code_nibble(uint32_t wbits, const RowScale &rs)
{
    return code_nibble_f(half_bits_to_float((uint16_t)wbits), rs.inv);
}

__device__ __forceinline__ uint32_t code_byte(uint32_t wbits, const RowScale &rs)
{
    return code_byte_f(half_bits_to_float((uint16_t)wbits), rs.inv);
}

// Eight INT8 codes of one 16-byte chunk as two dwords (element e in byte
// e % 4 of dword e / 4).
__device__ __forceinline__ uint2 bytes_chunk(u32x4 v, float inv)
{
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j / 2] |= code_byte_f(half_bits_to_float((uint16_t)(v[j] & 0xFFFFu)), inv) << (16 * (j % 2));
        o[j / 2] |= code_byte_f(half_bits_to_float((uint16_t)(v[j] >> 16)), inv) << (16 * (j % 2) + 8);
    }
    return uint2{o[0], o[1]};
}

// Eight codes of one 16-byte chunk (4 dwords of fp16 pairs) as one packed
// dword: element 2j in the low nibble of byte j, 2j + 1 in its high nibble.
__device__ __forceinline__ uint32_t pack_chunk(u32x4 v, float inv)
{
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        out |= code_nibble_f(half_bits_to_float((uint16_t)(v[j] & 0xFFFFu)), inv) << (8 * j);
        out |= code_nibble_f(half_bits_to_float((uint16_t)(v[j] >> 16)), inv) << (8 * j + 4);
    }
    return out;
}

// Register-resident path: WPR wavefronts per row, CH 16-byte chunks per lane
// (rows of up to 512 WPR CH halves).  Chunk c of wave part p of the row is
// chunk (c WPR + p) 64 + lane, so every load and store instruction covers
// consecutive memory.  Requires k % 8 == 0.
template <int WPR, int CH, int QMAX>
__global__ __launch_bounds__(kQThreads) void quantize_rows_reg(const uint16_t *__restrict__ w,
                                                               int64_t n, int64_t k,
                                                               uint8_t *__restrict__ packed,
                                                               uint16_t *__restrict__ scales)
{
    constexpr int RPW = (kQThreads / kWave) / WPR;          // rows per workgroup
    __shared__ uint32_t lds4[kQThreads / kWave];
    const int lane = threadIdx.x % kWave;
    // uniform: keeps the row's buffer descriptor in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int part = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPW + wave / WPR;
    const bool live = row < n;                             // uniform per wave
    const int64_t rowc = live ? row : n - 1;               // keeps the loads in range
    const int64_t nchunk = k / 8;
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(w + rowc * k, k * 2);

    u32x4 v[CH];
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t idx = ((int64_t)c * WPR + part) * kWave + lane;
        v[c] = buf_load16_stream(rs_w, idx < nchunk ? (uint32_t)(idx * 16) : kOutOfRange);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = max(m, v[c][j] & 0x7FFFu);
            m = max(m, (v[c][j] >> 16) & 0x7FFFu);
        }
    m = wave_max_u32(m);
    if (WPR > 1) {
        if (lane == 0)
            lds4[wave] = m;
        __syncthreads();
        const int w0 = wave - part;
#pragma unroll
        for (int p = 0; p < WPR; ++p)
            m = max(m, lds4[w0 + p]);
    }
    const RowScale rs = make_scale<QMAX>(m);
    if (live && part == 0 && lane == 0)
        scales[row] = rs.bits;
    if (!live)
        return;
    if constexpr (QMAX == 7) {
        uint32_t *pr = reinterpret_cast<uint32_t *>(packed + row * (k / 2));
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t idx = ((int64_t)c * WPR + part) * kWave + lane;
            if (idx < nchunk)
                pr[idx] = pack_chunk(v[c], rs.inv);
        }
    } else {
        uint2 *pr = reinterpret_cast<uint2 *>(packed + row * k);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t idx = ((int64_t)c * WPR + part) * kWave + lane;
            if (idx < nchunk)
                pr[idx] = bytes_chunk(v[c], rs.inv);
        }
    }
}

// General path (any even k, any row length): two sweeps over the row; the
// second one mostly hits in cache.
template <int QMAX>
__global__ __launch_bounds__(kQThreads) void quantize_rows_generic(const uint16_t *__restrict__ w,
                                                                   int64_t k,
                                                                   uint8_t *__restrict__ packed,
                                                                   uint16_t *__restrict__ scales)
{
    __shared__ uint32_t lds4[4];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * k;
    uint8_t *pr = packed + row * (QMAX == 7 ? k / 2 : k);
    const int64_t npair = k / 2;
    const uint32_t *wr2 = reinterpret_cast<const uint32_t *>(wr);   // k even: 4-byte pairs

    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < npair; i += kQThreads) {
        const uint32_t p = wr2[i];
        m = max(m, p & 0x7FFFu);
        m = max(m, (p >> 16) & 0x7FFFu);
    }
    const uint32_t amax = block_max_u32(m, lds4);
    const RowScale rs = make_scale<QMAX>(amax);
    if (threadIdx.x == 0)
        scales[row] = rs.bits;
    for (int64_t i = threadIdx.x; i < npair; i += kQThreads) {
        const uint32_t p = wr2[i];
        if constexpr (QMAX == 7)
            pr[i] = (uint8_t)(code_nibble(p & 0xFFFFu, rs) | (code_nibble(p >> 16, rs) << 4));
        else
            reinterpret_cast<uint16_t *>(pr)[i] =
                (uint16_t)(code_byte(p & 0xFFFFu, rs) | (code_byte(p >> 16, rs) << 8));
    }
}

template <int QMAX>
static hipError_t launch_quantize_q(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                                    hipStream_t stream)
{
    const uint16_t *wp = static_cast<const uint16_t *>(w);
    uint8_t *pp = static_cast<uint8_t *>(packed);
    uint16_t *sp = static_cast<uint16_t *>(scales);
    // lanes' chunks per row: at most 16 per lane, spread over 1, 2 or 4 waves
    const int64_t lane_chunks = (k / 8 + kWave - 1) / kWave;
#define W4_QREG(WPR, CH)                                                                           \
    hipLaunchKernelGGL((quantize_rows_reg<WPR, CH, QMAX>),                                         \
                       dim3((unsigned)((n + (4 / WPR) - 1) / (4 / WPR))), dim3(kQThreads), 0,       \
                       stream, wp, n, k, pp, sp)
    if (k % 8 == 0 && lane_chunks <= 64) {
        if (lane_chunks <= 1)
            W4_QREG(1, 1);
        else if (lane_chunks <= 2)
            W4_QREG(1, 2);
        else if (lane_chunks <= 4)
            W4_QREG(1, 4);
        else if (lane_chunks <= 8)
            W4_QREG(1, 8);
        else if (lane_chunks <= 16)
            W4_QREG(1, 16);
        else if (lane_chunks <= 24)
            W4_QREG(2, 12);
        else if (lane_chunks <= 32)
            W4_QREG(2, 16);
        else if (lane_chunks <= 48)
            W4_QREG(4, 12);
        else
            W4_QREG(4, 16);
    } else {
        hipLaunchKernelGGL(quantize_rows_generic<QMAX>, dim3((unsigned)n), dim3(kQThreads), 0,
                           stream, wp, k, pp, sp);
    }
#undef W4_QREG
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Zero-point INT4 variant (the pages' comparison scheme; the formula is the
// standard asymmetric 4-bit one):
//   lo = min(min_c W, 0), hi = max(max_c W, 0)
//   s  = fp16((hi - lo) / 15),  z = clamp(round_half_even(-lo / s), 0, 15)
//   q  = clamp(round_half_even(W / s) + z, 0, 15)   (unsigned nibbles)
// One 256-thread workgroup per row, two sweeps (the second hits in cache).
// Exactness: hi - lo is exact in binary64 (it can need up to 40 significant
// bits) and the division is correctly rounded.  The binary64 quotient is
// then rounded to fp16 once (half_bits_of_double): converting it to fp32
// with ties to even and then to fp16 would round twice, and that is not
// harmless here because the dividend has more than 11 significant bits
// (row [1934, -0.0624694824, 0, ...]: the quotient 128.9374980 lands on the
// fp32 value 128.9375, an fp16 tie, which then goes up to 129 instead of
// down to 128.875).  The binary64 quotient itself is the correctly rounded
// fp16 quotient's source: a non-midpoint quotient of a multiple of 2^-24 by
// 15 lies at least 2^-24 / 15 from every fp16 midpoint, far more than a
// binary64 rounding moves it.  -lo / s in binary64 is
// far closer to the exact quotient than the 2^-12 gap that separates a
// non-tie quotient from a half-integer, so rint gives its round-half-even.
// The codes follow the INT4 steps (|w / s| <= 15 here).
// ---------------------------------------------------------------------------
// fp16 bits of a finite binary64 value, rounded once (to nearest, ties to
// even).  The value goes to fp32 by round-to-odd (the nearest fp32, stepped
// back towards zero if it rounded away, with its last bit set whenever the
// conversion was inexact), which keeps enough of the dropped part for the
// final fp32 -> fp16 rounding to be the correctly rounded one: 24 >= 11 + 2
// bits.  fp16 results that are subnormal keep fewer bits, so the margin only
// grows.
__device__ __forceinline__ uint16_t half_bits_of_double(double d)
{
    const float f = (float)d;
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    const double back = (double)f;
    if (back != d) {
        if (__builtin_fabs(back) > __builtin_fabs(d))
            b -= 1u;                    // sign-magnitude: one step towards zero
        b |= 1u;
    }
    return float_to_half_bits(__builtin_bit_cast(float, b));
}

__device__ __forceinline__ uint32_t code_zp_f(float wf, float inv, float zf)
{
    const float r = wf * inv;
    const float snap = __fsub_rn(__fadd_rn(r, 3072.0f), 3072.0f);
    return (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(snap) + zf, 0.0f, 15.0f);
}

__global__ __launch_bounds__(kQThreads) void quantize_rows_zp(const uint16_t *__restrict__ w,
                                                              int64_t k,
                                                              uint8_t *__restrict__ packed,
                                                              uint16_t *__restrict__ scales,
                                                              uint8_t *__restrict__ zeros)
{
    __shared__ float red[2][kQThreads / kWave];
    const int64_t row = blockIdx.x;
    const uint16_t *wr = w + row * k;
    uint8_t *pr = packed + row * (k / 2);
    const bool chunks = k % 8 == 0;                 // 16-byte loads, 4-byte stores
    const int64_t nchunk = chunks ? k / 8 : k / 2;

    float lo = 0.0f, hi = 0.0f;
    for (int64_t i = threadIdx.x; i < nchunk; i += kQThreads) {
        if (chunks) {
            const u32x4 v = load16(wr + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = half_bits_to_float((uint16_t)(v[j] & 0xFFFFu));
                const float b = half_bits_to_float((uint16_t)(v[j] >> 16));
                lo = fminf(lo, fminf(a, b));
                hi = fmaxf(hi, fmaxf(a, b));
            }
        } else {
            const uint32_t p2 = reinterpret_cast<const uint32_t *>(wr)[i];
            const float a = half_bits_to_float((uint16_t)(p2 & 0xFFFFu));
            const float b = half_bits_to_float((uint16_t)(p2 >> 16));
            lo = fminf(lo, fminf(a, b));
            hi = fmaxf(hi, fmaxf(a, b));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
    }
    const int wave = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQThreads / kWave; ++i) {
        lo = fminf(lo, red[0][i]);
        hi = fmaxf(hi, red[1][i]);
    }
    const uint16_t sb = half_bits_of_double(((double)hi - (double)lo) / 15.0);
    const float s = half_bits_to_float(sb);
    float inv = 0.0f, zf = 0.0f;
    if (s != 0.0f) {
        inv = __fdiv_rn(1.0f, s);
        zf = (float)__builtin_rint(-(double)lo / (double)s);
        zf = __builtin_amdgcn_fmed3f(zf, 0.0f, 15.0f);
    }
    if (threadIdx.x == 0) {
        scales[row] = sb;
        zeros[row] = (uint8_t)zf;
    }
    for (int64_t i = threadIdx.x; i < nchunk; i += kQThreads) {
        if (chunks) {
            const u32x4 v = load16(wr + 8 * i);
            uint32_t out = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out |= code_zp_f(half_bits_to_float((uint16_t)(v[j] & 0xFFFFu)), inv, zf) << (8 * j);
                out |= code_zp_f(half_bits_to_float((uint16_t)(v[j] >> 16)), inv, zf) << (8 * j + 4);
            }
            reinterpret_cast<uint32_t *>(pr)[i] = out;
        } else {
            const uint32_t p2 = reinterpret_cast<const uint32_t *>(wr)[i];
            pr[i] = (uint8_t)(code_zp_f(half_bits_to_float((uint16_t)(p2 & 0xFFFFu)), inv, zf) |
                              (code_zp_f(half_bits_to_float((uint16_t)(p2 >> 16)), inv, zf) << 4));
        }
    }
}

// Register-resident zero-point path (k % 8 == 0, rows up to 512 WPR CH
// halves): the layout of quantize_rows_reg, with the row's min and max
// reduced instead of its absmax, so HBM is read once.
template <int WPR, int CH>
__global__ __launch_bounds__(kQThreads) void quantize_rows_zp_reg(const uint16_t *__restrict__ w,
                                                                  int64_t n, int64_t k,
                                                                  uint8_t *__restrict__ packed,
                                                                  uint16_t *__restrict__ scales,
                                                                  uint8_t *__restrict__ zeros)
{
    constexpr int RPW = (kQThreads / kWave) / WPR;          // rows per workgroup
    __shared__ float red[2][kQThreads / kWave];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int part = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPW + wave / WPR;
    const bool live = row < n;
    const int64_t rowc = live ? row : n - 1;
    const int64_t nchunk = k / 8;
    const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(w + rowc * k, k * 2);

    u32x4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t idx = ((int64_t)c * WPR + part) * kWave + lane;
        v[c] = buf_load16_stream(rs_w, idx < nchunk ? (uint32_t)(idx * 16) : kOutOfRange);
    }
    // chunks past the row read zeros, which min(., 0) and max(., 0) absorb
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = half_bits_to_float((uint16_t)(v[c][j] & 0xFFFFu));
            const float b = half_bits_to_float((uint16_t)(v[c][j] >> 16));
            lo = fminf(lo, fminf(a, b));
            hi = fmaxf(hi, fmaxf(a, b));
        }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
    }
    if (WPR > 1) {
        if (lane == 0) {
            red[0][wave] = lo;
            red[1][wave] = hi;
        }
        __syncthreads();
        const int w0 = wave - part;
#pragma unroll
        for (int p = 0; p < WPR; ++p) {
            lo = fminf(lo, red[0][w0 + p]);
            hi = fmaxf(hi, red[1][w0 + p]);
        }
    }
    const uint16_t sb = half_bits_of_double(((double)hi - (double)lo) / 15.0);
    const float sf = half_bits_to_float(sb);
    float inv = 0.0f, zf = 0.0f;
    if (sf != 0.0f) {
        inv = __fdiv_rn(1.0f, sf);
        zf = __builtin_amdgcn_fmed3f((float)__builtin_rint(-(double)lo / (double)sf), 0.0f, 15.0f);
    }
    if (live && part == 0 && lane == 0) {
        scales[row] = sb;
        zeros[row] = (uint8_t)zf;
    }
    if (!live)
        return;
    uint32_t *pr = reinterpret_cast<uint32_t *>(packed + row * (k / 2));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t idx = ((int64_t)c * WPR + part) * kWave + lane;
        if (idx < nchunk) {
            uint32_t out = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out |= code_zp_f(half_bits_to_float((uint16_t)(v[c][j] & 0xFFFFu)), inv, zf) << (8 * j);
                out |= code_zp_f(half_bits_to_float((uint16_t)(v[c][j] >> 16)), inv, zf) << (8 * j + 4);
            }
            pr[idx] = out;
        }
    }
}

hipError_t launch_quantize_zp(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                              void *zeros, hipStream_t stream)
{
    const uint16_t *wp = static_cast<const uint16_t *>(w);
    uint8_t *pp = static_cast<uint8_t *>(packed);
    uint16_t *sp = static_cast<uint16_t *>(scales);
    uint8_t *zp = static_cast<uint8_t *>(zeros);
    const int64_t lane_chunks = (k / 8 + kWave - 1) / kWave;
#define ZP_QREG(WPR, CH)                                                                           \
    hipLaunchKernelGGL((quantize_rows_zp_reg<WPR, CH>),                                            \
                       dim3((unsigned)((n + (4 / WPR) - 1) / (4 / WPR))), dim3(kQThreads), 0,       \
                       stream, wp, n, k, pp, sp, zp)
    if (k % 8 == 0 && lane_chunks <= 64) {
        if (lane_chunks <= 4)
            ZP_QREG(1, 4);
        else if (lane_chunks <= 8)
            ZP_QREG(1, 8);
        else if (lane_chunks <= 16)
            ZP_QREG(1, 16);
        else if (lane_chunks <= 32)
            ZP_QREG(2, 16);
        else
            ZP_QREG(4, 16);
    } else {
        hipLaunchKernelGGL(quantize_rows_zp, dim3((unsigned)n), dim3(kQThreads), 0, stream, wp, k, pp,
                           sp, zp);
    }
#undef ZP_QREG
    return hipGetLastError();
}

hipError_t launch_quantize(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                           hipStream_t stream)
{
    return launch_quantize_q<7>(w, n, k, packed, scales, stream);
}

hipError_t launch_quantize_int8(const void *w, int64_t n, int64_t k, void *codes, void *scales,
                                hipStream_t stream)
{
    return launch_quantize_q<127>(w, n, k, codes, scales, stream);
}

}  // namespace w4a16
