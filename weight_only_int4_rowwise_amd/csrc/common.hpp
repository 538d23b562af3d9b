// Device helpers shared by the gfx950 kernels of the W4A16 library.
//
// Packed weight layout (include/w4a16.h): uint8 [n][k/2], code 2j in the low
// nibble of byte j, code 2j+1 in the high nibble, 4-bit two's complement,
// codes in [-7, 7] (GLM-130B paper card, "Method" and "Paper vs code":
// two INT4 values per byte, integers in [-7, 7]).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// INT4 -> FP16 dequantization of one dword (8 codes) into one MFMA operand.
//
// Flipping bit 3 of each nibble turns the two's-complement code q into the
// offset-binary u = q + 8 in [1, 15].  OR-ing u into the mantissa of a
// binary16 with a fixed exponent gives an exact value:
//   0x6400 | u         = 1024 + u   (mantissa ulp 1 at exponent 10)
//   0x5400 | (u << 4)  =   64 + u   (mantissa bit 4 worth 1 at exponent 6)
// so one AND-OR forms two halves, and one packed f16 subtract of 1032 or 72
// returns q exactly.  The four packed dwords hold the codes of byte offsets
// (k0,k4) (k1,k5) (k2,k6) (k3,k7): element e of the operand is code
// kPerm[e] of the dword.  The other operand is permuted the same way, and
// since a dot product does not depend on the order of its terms the result
// is unchanged.
// ---------------------------------------------------------------------------
__device__ constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};

__device__ __forceinline__ half2v bits_to_h2(uint32_t v)
{
    return __builtin_bit_cast(half2v, v);
}

__device__ __forceinline__ half8 dequant8(uint32_t packed)
{
    const uint32_t u = packed ^ 0x88888888u;
    const uint32_t u8 = u >> 8;
    const half2v lo_bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v hi_bias = {(_Float16)72.0f, (_Float16)72.0f};
    half2v p0 = bits_to_h2((u & 0x000F000Fu) | 0x64006400u) - lo_bias;   // k0, k4
    half2v p1 = bits_to_h2((u & 0x00F000F0u) | 0x54005400u) - hi_bias;   // k1, k5
    half2v p2 = bits_to_h2((u8 & 0x000F000Fu) | 0x64006400u) - lo_bias;  // k2, k6
    half2v p3 = bits_to_h2((u8 & 0x00F000F0u) | 0x54005400u) - hi_bias;  // k3, k7
    half8 r;
    r[0] = p0[0]; r[1] = p0[1];
    r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1];
    r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Eight consecutive fp16 activations (as four dwords, natural order) into
// the operand order kPerm that matches dequant8.
__device__ __forceinline__ u32x4 permute_x8(u32x4 d)
{
    u32x4 p;
    p[0] = (d[0] & 0xFFFFu) | (d[2] << 16);          // x0, x4
    p[1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);      // x1, x5
    p[2] = (d[1] & 0xFFFFu) | (d[3] << 16);          // x2, x6
    p[3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);      // x3, x7
    return p;
}

__device__ __forceinline__ half8 as_half8(u32x4 v)
{
    return __builtin_bit_cast(half8, v);
}

// D = A * B + C on a 16 x 16 x 32 fp16 tile with fp32 accumulation.
// Lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16]
// for e = 0..7 and receives D[4 (l / 16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ float4v mfma16x16x32(half8 a, half8 b, float4v c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Streaming 16-byte load that is not kept in the caches (weights are read
// once per call; keeping them out of L2 leaves room for the activations).
__device__ __forceinline__ u32x4 load_stream16(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);   // round to nearest even
}

// GELU in its defining form t * Phi(t) = t/2 * (1 + erf(t / sqrt 2)), with
// the device math library's erff.
__device__ __forceinline__ float gelu_erf(float t)
{
    return 0.5f * t * (1.0f + erff(t * 0.70710678118654752440f));
}

}  // namespace w4a16
