// C ABI of the W4A16 library and its W8A16 variant: argument checks,
// kernel selection, error mapping.  Contract and citations: include/w4a16.h
// and include/w8a16.h.
#include "../../include/w4a16.h"
#include "../../include/w8a16.h"
#include "../../include/w4a16_zp.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace w4a16 {
hipError_t launch_quantize(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                           hipStream_t stream);
hipError_t launch_quantize_int8(const void *w, int64_t n, int64_t k, void *codes, void *scales,
                                hipStream_t stream);
hipError_t launch_quantize_zp(const void *w, int64_t n, int64_t k, void *packed, void *scales,
                              void *zeros, hipStream_t stream);
hipError_t launch_decode(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, const void *zeros, void *y, bool geglu,
                         bool tiled, int cb, hipStream_t stream);
hipError_t launch_prefill(const void *x, int64_t m, int64_t k, const void *packed,
                          const void *scales, int64_t n_out, const void *bias, const void *zeros,
                          void *y, bool geglu, bool tiled, int cb, hipStream_t stream);
int64_t prepacked_bytes(int64_t n, int64_t k);
hipError_t launch_prepack(const void *src, int64_t n, int64_t k, void *dst, hipStream_t stream);
int64_t prepacked_bytes_int8(int64_t n, int64_t k);
hipError_t launch_prepack_int8(const void *src, int64_t n, int64_t k, void *dst, hipStream_t stream);
hipError_t launch_read_probe(const void *src, int64_t bytes, void *sink, hipStream_t stream);
}  // namespace w4a16

namespace {

thread_local char g_last_error[256] = "";

// Largest dimension accepted: grids and in-kernel int arithmetic stay far
// from overflow, and the largest GLM-130B shapes (65536 rows, 32768 columns,
// 2048 tokens) fit with room to spare.
constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kDecodeMaxM = 64;
// Activations and weights must each stay below 2 GiB (32-bit buffer offsets).
constexpr int64_t kMaxBufferBytes = int64_t(1) << 31;

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

w4a16_status from_hip(hipError_t e)
{
    if (e == hipSuccess) {
        g_last_error[0] = '\0';
        return W4A16_OK;
    }
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction)
        return W4A16_ERR_DEVICE;
    return W4A16_ERR_HIP;
}

// Sizes first: an empty call (m == 0 or rows == 0) is valid whatever the
// pointers are (torch hands out NULL for empty tensors).
w4a16_status check_gemm_shape(int64_t m, int64_t k, int64_t rows, bool tiled, int cb)
{
    if (m < 0 || rows < 0 || k <= 0 || k % 32 != 0 || m > kMaxDim || rows > kMaxDim ||
        k > kMaxDim || m * k > (int64_t(1) << 40) || m * rows > (int64_t(1) << 40))
        return W4A16_ERR_SHAPE;
    // the kernels address the activations and the weight with 32-bit
    // buffer offsets
    const int64_t wbytes = cb == 8 ? (tiled ? w4a16::prepacked_bytes_int8(rows, k) : rows * k)
                                   : (tiled ? w4a16::prepacked_bytes(rows, k) : rows * (k / 2));
    if (2 * m * k >= kMaxBufferBytes || wbytes >= kMaxBufferBytes)
        return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

w4a16_status check_gemm_ptrs(const void *x, const void *q, const void *s, const void *bias,
                             const void *y)
{
    if (!x || !q || !s || !y)
        return W4A16_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s) || !aligned16(y) ||
        (bias && !aligned16(bias)))
        return W4A16_ERR_ALIGN;
    return W4A16_OK;
}

// 64 < m <= 128 runs the decode kernel twice (next function), unless one
// GEMM launch is faster: from the m this returns, by weight height in the
// decode kernel's own bands (the second decode launch gets slower as m - 64
// crosses its token classes, while the GEMM costs about the same anywhere in
// 64 < m <= 128) and, for 8192 to 16383 rows, by reduction length.  Measured
// on MI355X on the codes of quantized normal weights, prepacked, two decode
// launches against one GEMM launch (us):
//  * QKV 36864 x 12288 and plain 65536 x 12288: m = 112 115.3 / 122.5,
//    m = 120 125.5 / 122.9 (FFN-up 185.3 / 190.6, 195.5 / 190.7);
//  * 2-way QKV shard 18432 x 12288 (its M = 64 decode has 128 workgroups):
//    m = 65 76.0 / 71.5;
//  * 8192 to 16383 rows: k >= 8192 (attention-out 12288 x 12288, FFN-down
//    12288 x 32768 and its 2- and 4-way shards, 4-way QKV 9216 x 12288):
//    m = 80 52.1 / 53.2, m = 88 55.9 / 52.0 (attention-out); 4096 <= k
//    < 8192 (12288 x 6144, 12288 x 4096): m = 72 22.4 / 22.7, m = 80
//    23.4 / 22.7; k < 4096 (12288 x 3072, 12288 x 1536): m = 65 13.8 /
//    12.4 (k = 1536);
//  * fewer rows with a long reduction (8-way QKV 4608 x 12288): m = 96
//    47.6 / 50.8, m = 104 53.8 / 50.6;
//  * GeGLU FFN-up 65536 x 12288: m = 96 170.6 / 181.8, m = 104 to 112
//    even, m = 120 195.1 / 186.9; its 2-way shard (32768 rows): m = 65
//    119.9 / 103.9; 4-way (16384 rows): m = 96 67.8 / 68.8, m = 104 74.4 /
//    69.0; 8-way (8192 rows): two decode launches at every m (m = 128
//    62.1 / 66.1).
// Shapes below these bands keep two decode launches.  INT8 codes always do:
// their GEMM has no split-reduction tiles.
static int64_t gemm_from_m(int64_t k, int64_t rows, bool geglu)
{
    const int64_t never = 2 * kDecodeMaxM + 1;
    if (geglu)
        return rows >= 49152 ? 120 : rows >= 24576 ? 65 : rows >= 12288 ? 104 : never;
    if (rows >= 24576)
        return 120;
    if (rows >= 16384)
        return 65;
    if (rows >= 8192)
        return k >= 8192 ? 88 : k >= 4096 ? 80 : 65;
    return k >= 8192 ? 104 : never;
}

static bool gemm_beats_two_decodes(int64_t m, int64_t k, int64_t rows, bool geglu, int cb)
{
    return cb == 4 && m >= gemm_from_m(k, rows, geglu);
}

// zeros: per-row zero points of the zero-point INT4 variant, or NULL.
w4a16_status run_linear(const void *x, int64_t m, int64_t k, const void *q, const void *s,
                        int64_t n_out, const void *bias, void *y, bool geglu, bool tiled, int cb,
                        void *stream, const void *zeros = nullptr, bool zp = false)
{
    const int64_t rows = geglu ? 2 * n_out : n_out;
    w4a16_status st = check_gemm_shape(m, k, rows, tiled, cb);
    if (st != W4A16_OK)
        return st;
    if (m == 0 || n_out == 0)
        return W4A16_OK;
    st = check_gemm_ptrs(x, q, s, bias, y);
    if (st != W4A16_OK)
        return st;
    if (zp && !zeros)
        return W4A16_ERR_NULL;
    if (zp && !aligned16(zeros))
        return W4A16_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (m <= kDecodeMaxM) {
        e = w4a16::launch_decode(x, (int)m, k, q, s, n_out, bias, zeros, y, geglu, tiled, cb, hs);
    } else if (m <= 2 * kDecodeMaxM && !gemm_beats_two_decodes(m, k, rows, geglu, cb)) {
        // 64 < m <= 128: the first 64 tokens, then the rest, each through
        // the decode kernel.  The weights stream twice, but every CU stays
        // busy, where the GEMM's tiles leave most of the chip idle at this
        // size (FFN-down 12288 x 32768 at m = 65: 122 against 207 us;
        // attention-out 12288 x 12288 at m = 96: 59 against 83 us).
        // Outputs depend only on their own token row, so the split changes
        // no result bits.
        e = w4a16::launch_decode(x, (int)kDecodeMaxM, k, q, s, n_out, bias, zeros, y, geglu, tiled,
                                 cb, hs);
        if (e == hipSuccess)
            e = w4a16::launch_decode(static_cast<const uint16_t *>(x) + kDecodeMaxM * k,
                                     (int)(m - kDecodeMaxM), k, q, s, n_out, bias, zeros,
                                     static_cast<uint16_t *>(y) + kDecodeMaxM * n_out, geglu,
                                     tiled, cb, hs);
    } else {
        e = w4a16::launch_prefill(x, m, k, q, s, n_out, bias, zeros, y, geglu, tiled, cb, hs);
    }
    return from_hip(e);
}

}  // namespace

extern "C" {

w4a16_status quantize_rowwise_int4(const void *w_fp16, int64_t n, int64_t k, void *q_packed,
                                   void *scales_fp16, void *stream)
{
    if (n < 0 || k < 2 || k % 2 != 0 || n > 0x7FFFFFFF || k > kMaxDim)
        return W4A16_ERR_SHAPE;
    if (n == 0)
        return W4A16_OK;
    if (!w_fp16 || !q_packed || !scales_fp16)
        return W4A16_ERR_NULL;
    if (!aligned16(w_fp16) || !aligned16(q_packed) || !aligned16(scales_fp16))
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_quantize(w_fp16, n, k, q_packed, scales_fp16,
                                           static_cast<hipStream_t>(stream)));
}

w4a16_status w4a16_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                          const void *scales_fp16, int64_t n, const void *bias_fp16, void *y_fp16,
                          void *stream)
{
    return run_linear(x_fp16, m, k, q_packed, scales_fp16, n, bias_fp16, y_fp16, false, false, 4,
                      stream);
}

w4a16_status w4a16_geglu_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                                const void *scales_fp16, int64_t f, const void *bias_fp16,
                                void *y_fp16, void *stream)
{
    if (f > kMaxDim / 2)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, q_packed, scales_fp16, f, bias_fp16, y_fp16, true, false, 4,
                      stream);
}

int64_t w4a16_prepacked_bytes(int64_t n, int64_t k)
{
    if (n < 0 || k <= 0 || k % 32 != 0 || n > kMaxDim || k > kMaxDim)
        return -1;
    return w4a16::prepacked_bytes(n, k);
}

w4a16_status w4a16_prepack(const void *q_packed, int64_t n, int64_t k, void *q_prepacked,
                           void *stream)
{
    if (w4a16_prepacked_bytes(n, k) < 0)
        return W4A16_ERR_SHAPE;
    if (n == 0)
        return W4A16_OK;
    if (!q_packed || !q_prepacked)
        return W4A16_ERR_NULL;
    if (!aligned16(q_packed) || !aligned16(q_prepacked))
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_prepack(q_packed, n, k, q_prepacked,
                                          static_cast<hipStream_t>(stream)));
}

w4a16_status w4a16_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                    const void *q_prepacked, const void *scales_fp16, int64_t n,
                                    const void *bias_fp16, void *y_fp16, void *stream)
{
    return run_linear(x_fp16, m, k, q_prepacked, scales_fp16, n, bias_fp16, y_fp16, false, true, 4,
                      stream);
}

w4a16_status w4a16_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                          const void *q_prepacked, const void *scales_fp16,
                                          int64_t f, const void *bias_fp16, void *y_fp16,
                                          void *stream)
{
    // the gate / value boundary must fall on a 16-row tile boundary
    if (f > kMaxDim / 2 || f % 16 != 0)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, q_prepacked, scales_fp16, f, bias_fp16, y_fp16, true, true, 4,
                      stream);
}

w4a16_status quantize_rowwise_int8(const void *w_fp16, int64_t n, int64_t k, void *codes_i8,
                                   void *scales_fp16, void *stream)
{
    if (n < 0 || k < 2 || k % 2 != 0 || n > 0x7FFFFFFF || k > kMaxDim)
        return W4A16_ERR_SHAPE;
    if (n == 0)
        return W4A16_OK;
    if (!w_fp16 || !codes_i8 || !scales_fp16)
        return W4A16_ERR_NULL;
    if (!aligned16(w_fp16) || !aligned16(codes_i8) || !aligned16(scales_fp16))
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_quantize_int8(w_fp16, n, k, codes_i8, scales_fp16,
                                                static_cast<hipStream_t>(stream)));
}

w4a16_status w8a16_linear(const void *x_fp16, int64_t m, int64_t k, const void *codes_i8,
                          const void *scales_fp16, int64_t n, const void *bias_fp16, void *y_fp16,
                          void *stream)
{
    return run_linear(x_fp16, m, k, codes_i8, scales_fp16, n, bias_fp16, y_fp16, false, false, 8,
                      stream);
}

w4a16_status w8a16_geglu_linear(const void *x_fp16, int64_t m, int64_t k, const void *codes_i8,
                                const void *scales_fp16, int64_t f, const void *bias_fp16,
                                void *y_fp16, void *stream)
{
    if (f > kMaxDim / 2)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, codes_i8, scales_fp16, f, bias_fp16, y_fp16, true, false, 8,
                      stream);
}

int64_t w8a16_prepacked_bytes(int64_t n, int64_t k)
{
    if (n < 0 || k <= 0 || k % 32 != 0 || n > kMaxDim || k > kMaxDim)
        return -1;
    return w4a16::prepacked_bytes_int8(n, k);
}

w4a16_status w8a16_prepack(const void *codes_i8, int64_t n, int64_t k, void *codes_prepacked,
                           void *stream)
{
    if (w8a16_prepacked_bytes(n, k) < 0)
        return W4A16_ERR_SHAPE;
    if (n == 0)
        return W4A16_OK;
    if (!codes_i8 || !codes_prepacked)
        return W4A16_ERR_NULL;
    if (!aligned16(codes_i8) || !aligned16(codes_prepacked))
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_prepack_int8(codes_i8, n, k, codes_prepacked,
                                               static_cast<hipStream_t>(stream)));
}

w4a16_status w8a16_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                    const void *codes_prepacked, const void *scales_fp16, int64_t n,
                                    const void *bias_fp16, void *y_fp16, void *stream)
{
    return run_linear(x_fp16, m, k, codes_prepacked, scales_fp16, n, bias_fp16, y_fp16, false, true,
                      8, stream);
}

w4a16_status w8a16_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                          const void *codes_prepacked, const void *scales_fp16,
                                          int64_t f, const void *bias_fp16, void *y_fp16,
                                          void *stream)
{
    // the gate / value boundary must fall on a 16-row tile boundary
    if (f > kMaxDim / 2 || f % 16 != 0)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, codes_prepacked, scales_fp16, f, bias_fp16, y_fp16, true, true,
                      8, stream);
}

w4a16_status quantize_rowwise_int4_zp(const void *w_fp16, int64_t n, int64_t k, void *q_packed,
                                      void *scales_fp16, void *zeros_u8, void *stream)
{
    if (n < 0 || k < 2 || k % 2 != 0 || n > 0x7FFFFFFF || k > kMaxDim)
        return W4A16_ERR_SHAPE;
    if (n == 0)
        return W4A16_OK;
    if (!w_fp16 || !q_packed || !scales_fp16 || !zeros_u8)
        return W4A16_ERR_NULL;
    if (!aligned16(w_fp16) || !aligned16(q_packed) || !aligned16(scales_fp16) || !aligned16(zeros_u8))
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_quantize_zp(w_fp16, n, k, q_packed, scales_fp16, zeros_u8,
                                              static_cast<hipStream_t>(stream)));
}

w4a16_status w4a16_zp_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                             const void *scales_fp16, const void *zeros_u8, int64_t n,
                             const void *bias_fp16, void *y_fp16, void *stream)
{
    return run_linear(x_fp16, m, k, q_packed, scales_fp16, n, bias_fp16, y_fp16, false, false, 4,
                      stream, zeros_u8, true);
}

w4a16_status w4a16_zp_geglu_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                                   const void *scales_fp16, const void *zeros_u8, int64_t f,
                                   const void *bias_fp16, void *y_fp16, void *stream)
{
    if (f > kMaxDim / 2)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, q_packed, scales_fp16, f, bias_fp16, y_fp16, true, false, 4,
                      stream, zeros_u8, true);
}

w4a16_status w4a16_zp_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                       const void *q_prepacked, const void *scales_fp16,
                                       const void *zeros_u8, int64_t n, const void *bias_fp16,
                                       void *y_fp16, void *stream)
{
    return run_linear(x_fp16, m, k, q_prepacked, scales_fp16, n, bias_fp16, y_fp16, false, true, 4,
                      stream, zeros_u8, true);
}

w4a16_status w4a16_zp_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                             const void *q_prepacked, const void *scales_fp16,
                                             const void *zeros_u8, int64_t f,
                                             const void *bias_fp16, void *y_fp16, void *stream)
{
    if (f > kMaxDim / 2 || f % 16 != 0)
        return W4A16_ERR_SHAPE;
    return run_linear(x_fp16, m, k, q_prepacked, scales_fp16, f, bias_fp16, y_fp16, true, true, 4,
                      stream, zeros_u8, true);
}

w4a16_status w4a16_read_probe(const void *src, int64_t bytes, void *sink_u32, void *stream)
{
    if (bytes < 0 || bytes % 1024 != 0 || bytes > (int64_t(1) << 40))
        return W4A16_ERR_SHAPE;
    if (bytes == 0)
        return W4A16_OK;
    if (!src || !sink_u32)
        return W4A16_ERR_NULL;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink_u32) & 3u) != 0)
        return W4A16_ERR_ALIGN;
    return from_hip(w4a16::launch_read_probe(src, bytes, sink_u32, static_cast<hipStream_t>(stream)));
}

const char *w4a16_status_string(int status)
{
    switch (status) {
    case W4A16_OK:
        return "ok";
    case W4A16_ERR_NULL:
        return "a required pointer is NULL";
    case W4A16_ERR_SHAPE:
        return "invalid shape (negative size, k = 0, k not even for quantize, k % 32 != 0 for the "
               "linears, or size too large)";
    case W4A16_ERR_ALIGN:
        return "a pointer is not 16-byte aligned";
    case W4A16_ERR_HIP:
        return "HIP runtime error";
    case W4A16_ERR_DEVICE:
        return "no gfx950 code for the current device";
    default:
        return "unknown status";
    }
}

const char *w4a16_last_error(void)
{
    return g_last_error;
}

int w4a16_abi_version(void)
{
    return W4A16_ABI_VERSION;
}

}  // extern "C"
