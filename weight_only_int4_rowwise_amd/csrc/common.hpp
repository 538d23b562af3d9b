// Device helpers shared by the gfx950 kernels of the W4A16 library (and of
// its INT8 variant, W8A16: one two's-complement code per byte, [n][k]).
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
// INT4 -> FP16 dequantization of one dword (8 codes) into one MFMA operand
// holding the 8 codes in their natural order.
//
// Flipping bit 3 of a nibble turns the two's-complement code q into the
// offset-binary u = q + 8 in [1, 15].  Placing u in the mantissa of a
// binary16 with a fixed exponent gives an exact value:
//   0x6400 | u         = 1024 + u   (mantissa ulp 1 at exponent 10)
//   0x5400 | (u << 4)  =   64 + u   (mantissa bit 4 worth 1 at exponent 6)
// and one packed f16 subtract of 1032 or 72 returns q exactly.  The flip,
// the nibble mask and the exponent bits fold into one 3-input bit op:
//   ((w ^ 0x8888...) & M) | C  ==  (w & M) ^ B,   B = (0x8888... & M) | C
// since C has no bits inside M.
//
// dequant8 reads the prepacked nibble order, in which the dword of codes
// e0..e7 holds bytes (e0 | e2 << 4), (e4 | e6 << 4), (e1 | e3 << 4),
// (e5 | e7 << 4): the half pairs (e0,e1) (e2,e3) (e4,e5) (e6,e7) are then
// the low nibbles of bytes 0 and 2, their high nibbles, and the same for
// bytes 1 and 3.  9 VALU ops: one shift, four v_bitop3_b32, four
// v_pk_add_f16.
//
// dequant8_rm reads the row-major order of the pages' packing (byte i =
// e_2i | e_2i+1 << 4): one v_perm_b32 copies byte i into both halves, then
// its low nibble is e_2i in the low half and its high nibble e_2i+1 in the
// high half.  12 VALU ops.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v bits_to_h2(uint32_t v)
{
    return __builtin_bit_cast(half2v, v);
}

__device__ __forceinline__ half8 dequant8(uint32_t packed)
{
    const uint32_t w8 = packed >> 8;
    const half2v lo_bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v hi_bias = {(_Float16)72.0f, (_Float16)72.0f};
    // low nibbles: mask 0x000F000F, exponent 0x6400, flip 0x0008
    // high nibbles: mask 0x00F000F0, exponent 0x5400, flip 0x0080
    const half2v p0 = bits_to_h2((packed & 0x000F000Fu) ^ 0x64086408u) - lo_bias;   // e0, e1
    const half2v p1 = bits_to_h2((packed & 0x00F000F0u) ^ 0x54805480u) - hi_bias;   // e2, e3
    const half2v p2 = bits_to_h2((w8 & 0x000F000Fu) ^ 0x64086408u) - lo_bias;       // e4, e5
    const half2v p3 = bits_to_h2((w8 & 0x00F000F0u) ^ 0x54805480u) - hi_bias;       // e6, e7
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, p0);
    r[1] = __builtin_bit_cast(uint32_t, p1);
    r[2] = __builtin_bit_cast(uint32_t, p2);
    r[3] = __builtin_bit_cast(uint32_t, p3);
    return __builtin_bit_cast(half8, r);
}

__device__ __forceinline__ half8 dequant8_rm(uint32_t packed)
{
    const half2v bias = {(_Float16)1032.0f, (_Float16)72.0f};
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // byte i into bits [7:0] and [23:16], zeros elsewhere (selector 0x0c)
        const uint32_t sel = 0x0c000c00u | (uint32_t)i | ((uint32_t)i << 16);
        const uint32_t b = __builtin_amdgcn_perm(0u, packed, sel);
        const half2v p = bits_to_h2((b & 0x00F0000Fu) ^ 0x54806408u) - bias;
        r[i] = __builtin_bit_cast(uint32_t, p);
    }
    return __builtin_bit_cast(half8, r);
}

template <bool PREPACKED>
__device__ __forceinline__ half8 dequant8_of(uint32_t packed)
{
    return PREPACKED ? dequant8(packed) : dequant8_rm(packed);
}

// ---------------------------------------------------------------------------
// Zero-point INT4 -> FP16: unsigned codes u in [0, 15] and a per-row zero
// point z give the exact fp16 integers u - z in [-15, 15].  The bit trick of
// dequant8 without the sign flip puts 1024 + u (low nibbles) or 64 + u
// (high nibbles) in a binary16; the packed subtract then takes 1024 + z or
// 64 + z, held per lane for its row instead of as constants.  Same op count
// as dequant8 / dequant8_rm.
// ---------------------------------------------------------------------------
struct ZBias {
    half2v lo;   // (1024 + z, 1024 + z): low nibbles, prepacked order
    half2v hi;   // (64 + z, 64 + z): high nibbles, prepacked order
    half2v rm;   // (1024 + z, 64 + z): row-major order
};

// (w & m) ^ c as one v_bitop3_b32 (truth table 0x6a, index = 4 w + 2 m + c).
// With c disjoint from m the compiler rewrites the plain expression as an
// or, which it then emits as an and plus an or.
__device__ __forceinline__ uint32_t and_xor(uint32_t w, uint32_t m, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(w, m, c, 0x6a);
}

__device__ __forceinline__ ZBias make_zbias(uint32_t z)
{
    const _Float16 a = (_Float16)(1024.0f + (float)z), b = (_Float16)(64.0f + (float)z);
    return ZBias{half2v{a, a}, half2v{b, b}, half2v{a, b}};
}

__device__ __forceinline__ half8 dequant8_zp(uint32_t packed, const ZBias &zb)
{
    const uint32_t w8 = packed >> 8;
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, bits_to_h2(and_xor(packed, 0x000F000Fu, 0x64006400u)) - zb.lo);
    r[1] = __builtin_bit_cast(uint32_t, bits_to_h2(and_xor(packed, 0x00F000F0u, 0x54005400u)) - zb.hi);
    r[2] = __builtin_bit_cast(uint32_t, bits_to_h2(and_xor(w8, 0x000F000Fu, 0x64006400u)) - zb.lo);
    r[3] = __builtin_bit_cast(uint32_t, bits_to_h2(and_xor(w8, 0x00F000F0u, 0x54005400u)) - zb.hi);
    return __builtin_bit_cast(half8, r);
}

__device__ __forceinline__ half8 dequant8_rm_zp(uint32_t packed, const ZBias &zb)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t sel = 0x0c000c00u | (uint32_t)i | ((uint32_t)i << 16);
        const uint32_t b = __builtin_amdgcn_perm(0u, packed, sel);
        r[i] = __builtin_bit_cast(uint32_t, bits_to_h2(and_xor(b, 0x00F0000Fu, 0x54006400u)) - zb.rm);
    }
    return __builtin_bit_cast(half8, r);
}

template <bool PREPACKED>
__device__ __forceinline__ half8 dequant8_zp_of(uint32_t packed, const ZBias &zb)
{
    return PREPACKED ? dequant8_zp(packed, zb) : dequant8_rm_zp(packed, zb);
}

// ---------------------------------------------------------------------------
// INT8 -> FP16 dequantization of two dwords (8 codes in their natural
// order) into one MFMA operand.  A code q in [-127, 127] as the offset
// byte u = q + 128 (q's two's-complement byte with its top bit flipped)
// under the exponent byte 0x64 is the binary16 1024 + u, exact; one packed
// f16 subtract of 1152 returns q.  One v_perm_b32 builds two such halves
// from two code bytes and a constant 0x64 byte (selector bytes 0..3 pick
// the code dword, 4 picks the constant).  The prepacked layout stores the
// offset bytes (8 VALU ops per 8 codes); the row-major one stores two's
// complement and adds one xor per dword (10 ops).
// ---------------------------------------------------------------------------
__device__ __forceinline__ half8 dequant8_i8(uint32_t lo, uint32_t hi)
{
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, bits_to_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - bias);
    r[1] = __builtin_bit_cast(uint32_t, bits_to_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - bias);
    r[2] = __builtin_bit_cast(uint32_t, bits_to_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - bias);
    r[3] = __builtin_bit_cast(uint32_t, bits_to_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - bias);
    return __builtin_bit_cast(half8, r);
}

template <bool PREPACKED>
__device__ __forceinline__ half8 dequant8_i8_of(uint32_t lo, uint32_t hi)
{
    if (!PREPACKED) {
        lo ^= 0x80808080u;
        hi ^= 0x80808080u;
    }
    return dequant8_i8(lo, hi);
}

// Row-major packed dword -> the prepacked nibble order read by dequant8.
__host__ __device__ __forceinline__ uint32_t prepack_nibbles(uint32_t w)
{
    const uint32_t lo = w & 0x0F0F0F0Fu;          // e0 e2 e4 e6 in bytes 0..3
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // e1 e3 e5 e7
    const uint32_t lp = lo | (lo >> 4);           // byte 0 = e0|e2<<4, byte 2 = e4|e6<<4
    const uint32_t hp = hi | (hi >> 4);
    return (lp & 0xFFu) | ((lp >> 8) & 0xFF00u) | ((hp & 0xFFu) << 16) | ((hp << 8) & 0xFF000000u);
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

// ---------------------------------------------------------------------------
// Range-checked buffer loads.  A buffer resource carries the byte size of
// the tensor; a load whose 16 bytes lie past it returns zeros without
// touching memory.  Kernels point padding lanes (rows or reduction indices
// past the end) at kOutOfRange instead of branching around the load, so
// every load is unconditional and the compiler can keep loads of later
// pipeline stages in flight across the current one.  Offsets are 32-bit:
// the library rejects tensors of 2 GiB or more.
// ---------------------------------------------------------------------------
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    // dword 3 = 0x00020000: 32-bit data format, the raw (stride 0) buffer
    // setting for gfx9-family matrix-core GPUs
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// plain (cached) 16-byte load
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// streaming 16-byte load (non-temporal: weights are read once per call)
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (gfx9 encoding; expcnt and lgkmcnt left at their maximum).
constexpr int vmcnt_imm(int n)
{
    return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70;
}

// 16-byte range-checked buffer load written straight to LDS (gfx950 LDS
// DMA): lane l's 16 bytes land at lds + 16 l, so a wavefront fills 1 KB of
// consecutive LDS; lds must be the same for all lanes.  Completion is
// tracked by the vector-memory counter only, so a barrier that publishes
// the data must be preceded by a wait on that counter.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             (int)off, 0, 0, 0);
}

// Byte offset of the 16 packed bytes (32 codes, reduction indices
// [kc, kc + 32)) that lane `lane` of an MFMA A operand holds for weight
// `row`; the lane's row is row % 16 == lane % 16 and kc % 128 == 32 (lane / 16).
//  row-major layout: [n][k/2] bytes.
//  prepacked layout: 16-row x 128-index tiles of 1 KB, tiles ordered by row
//  group then by reduction position, lane l's 16 bytes at offset 16 l.
template <bool TILED>
__device__ __forceinline__ uint32_t piece_off(int64_t row, int64_t kc, int64_t row_bytes,
                                              int64_t tiles_per_group, int lane)
{
    if (TILED)
        return (uint32_t)(((row >> 4) * tiles_per_group + (kc >> 7)) * 1024 + 16 * lane);
    return (uint32_t)(row * row_bytes + (kc >> 1));
}

// Per-lane base offset of weight `row` (kOutOfRange for padding rows) and
// the offset step of the piece starting at reduction index kc, both 32-bit,
// so that piece offsets are one add and one select (no branches).
template <bool TILED>
__device__ __forceinline__ uint32_t row_base_off(int64_t row, int64_t row_bytes,
                                                 int64_t tiles_per_group, int lane)
{
    if (row < 0)
        return kOutOfRange;
    return TILED ? (uint32_t)((row >> 4) * tiles_per_group * 1024 + 16 * lane)
                 : (uint32_t)(row * row_bytes);
}

template <bool TILED>
__device__ __forceinline__ uint32_t piece_step_off(uint32_t kc)
{
    return TILED ? (kc >> 7) * 1024u : (kc >> 1);
}

// Bytes of a weight of `rows` rows in either layout.
__host__ __device__ __forceinline__ int64_t weight_bytes(bool tiled, int64_t rows, int64_t k)
{
    return tiled ? ((rows + 15) / 16) * ((k + 127) / 128) * 1024 : rows * (k / 2);
}

// The same for cb-bit codes (4: two per byte, 1 KB tiles; 8: one per byte,
// 2 KB tiles of 16 rows x 128 indices).
__host__ __device__ __forceinline__ int64_t code_weight_bytes(int cb, bool tiled, int64_t rows, int64_t k)
{
    return cb == 8 ? (tiled ? ((rows + 15) / 16) * ((k + 127) / 128) * 2048 : rows * k)
                   : weight_bytes(tiled, rows, k);
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

// An output's fp32 value to fp16 bits (round to nearest even) as a step of
// its own.  The empty asm keeps the compiler from folding the multiply-add
// that produced v into a mixed-precision instruction that rounds straight to
// fp16: it does so in some kernel shapes and not in others, which would make
// the rounding, and so the bits, depend on the launch shape and the weight
// layout.  Every epilogue rounds the fp32 result, then to fp16.
__device__ __forceinline__ uint16_t output_half_bits(float v)
{
    asm volatile("" : "+v"(v));
    return float_to_half_bits(v);
}

// GELU in its defining form t * Phi(t) = t/2 * (1 + erf(t / sqrt 2)), with
// the device math library's erff.
__device__ __forceinline__ float gelu_erf(float t)
{
    return 0.5f * t * (1.0f + erff(t * 0.70710678118654752440f));
}

}  // namespace w4a16
