// Decode kernels of the INT8 variant (W8A16): its launch table and entry.
#include "decode.hpp"

namespace w4a16 {

// INT8 launch shapes: the INT4 bands with the chunk halved (128 indices of
// one-byte codes are the bytes of 256 INT4 indices, so a wave's loads per
// round stay the same size) and two weight register sets in flight; the
// tallest GeGLU weights at 16 < m <= 32 take two row groups per wave.  The
// INT4 shapes would need up to twice the weight registers and spill.  The
// tallest GeGLU weights at m <= 4 take one row set of two groups over eight
// K-parts with two 128-code pieces per chunk (65536 x 12288 on quantized
// normal codes, alternating with the earlier four-row-set shape through the
// ABI: 122.1-123.3 against 126.0-127.0 us at m = 1).
template <bool GEGLU, bool TILED>
static hipError_t launch_decode_layout8(const void *x, int m, int64_t k, const void *packed,
                                        const void *scales, int64_t n_out, const void *bias,
                                        void *y, hipStream_t stream)
{
    const void *zeros = nullptr;
    constexpr bool ZP = false;
    constexpr int CB = 8;
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
#define W4_DEC(KU, RG, W, D, MB, MR, NGW)                                                      \
    launch_decode_e<KU, RG, W, D, MB, MR, NGW, GEGLU, TILED, CB, ZP>(x, m, k, packed, scales, n_out, \
                                                                     bias, zeros, y, stream)
    if constexpr (GEGLU) {
        const int b = rows >= 49152 ? 3 : rows >= 24576 ? 2 : rows >= 12288 ? 1 : 0;
        if (m <= 4)
            b == 3   ? W4_DEC(2, 1, 8, 2, 1, 4, 2)
            : b == 2 ? W4_DEC(1, 2, 4, 2, 1, 4, 2)
            : b == 1 ? W4_DEC(1, 1, 4, 2, 1, 4, 2)
                     : W4_DEC(1, 1, 8, 2, 1, 4, 2);
        else if (m <= 8)
            b == 3 ? W4_DEC(1, 4, 4, 2, 1, 8, 2)
            : b    ? W4_DEC(1, 2, 8, 2, 1, 8, 2)
                   : W4_DEC(1, 1, 8, 2, 1, 8, 2);
        else if (m <= 16)
            b == 3 ? W4_DEC(1, 8, 16, 2, 1, 16, 2)
            : b    ? W4_DEC(1, 2, 8, 2, 1, 16, 2)
                   : W4_DEC(1, 1, 8, 2, 1, 16, 2);
        else if (m <= 32)
            b == 3   ? W4_DEC(1, 4, 16, 2, 2, 32, 2)
            : b == 2 ? W4_DEC(1, 2, 4, 2, 2, 32, 4)
            : b == 1 ? W4_DEC(1, 2, 8, 2, 2, 32, 2)
                     : W4_DEC(1, 1, 4, 2, 2, 32, 2);
        else if (m <= 48)
            b == 3   ? W4_DEC(1, 4, 8, 2, 3, 48, 4)
            : b == 2 ? W4_DEC(1, 2, 4, 2, 3, 48, 4)
            : b == 1 ? W4_DEC(1, 1, 4, 2, 3, 48, 4)
                     : W4_DEC(1, 1, 4, 2, 3, 48, 2);
        else
            b == 3 ? W4_DEC(1, 8, 16, 2, 4, 64, 2)
            : b    ? W4_DEC(1, 2, 4, 2, 4, 64, 2)
                   : W4_DEC(1, 1, 4, 2, 4, 64, 2);
    } else {
        const int b = rows >= 49152 ? 4 : rows >= 24576 ? 3 : rows >= 16384 ? 2 : rows >= 8192 ? 1 : 0;
        if (m <= 4)
            b == 4   ? W4_DEC(1, 4, 4, 2, 1, 4, 1)
            : b == 3 ? W4_DEC(1, 3, 6, 2, 1, 4, 1)
            : b      ? W4_DEC(1, 1, 4, 2, 1, 4, 1)
                     : W4_DEC(1, 1, 8, 2, 1, 4, 1);
        else if (m <= 8)
            b == 4   ? W4_DEC(1, 4, 4, 2, 1, 8, 1)
            : b >= 2 ? W4_DEC(1, 1, 4, 2, 1, 8, 3)
            : b == 1 ? (k < 4096 ? W4_DEC(1, 1, 4, 2, 1, 8, 1) : W4_DEC(2, 3, 12, 2, 1, 8, 1))
                     : W4_DEC(1, 2, 8, 2, 1, 8, 1);
        else if (m <= 16)
            b == 4                           ? W4_DEC(1, 4, 4, 2, 1, 16, 2)
            : b == 3                         ? W4_DEC(1, 3, 12, 2, 1, 16, 3)
            : b == 2 || (b == 1 && k < 4096) ? W4_DEC(1, 1, 4, 2, 1, 16, 3)
            : b == 1                         ? W4_DEC(1, 1, 8, 2, 1, 16, 3)
                                             : W4_DEC(1, 2, 8, 2, 1, 16, 1);
        else if (m <= 32)
            b == 4   ? W4_DEC(1, 2, 4, 2, 2, 32, 4)
            : b >= 2 ? W4_DEC(1, 3, 12, 2, 2, 32, 3)
            : b == 1 ? (k <= 4096 ? W4_DEC(1, 2, 8, 2, 2, 32, 2) : W4_DEC(1, 1, 4, 2, 2, 32, 3))
                     : W4_DEC(1, 1, 4, 2, 2, 32, 2);
        else if (m <= 48)
            b == 4   ? W4_DEC(1, 4, 8, 2, 3, 48, 4)
            : b >= 2 ? W4_DEC(1, 3, 12, 2, 3, 48, 3)
            : b == 1 ? W4_DEC(1, 1, 4, 2, 3, 48, 3)
                     : W4_DEC(1, 1, 4, 2, 3, 48, 2);
        else
            b == 4   ? W4_DEC(1, 8, 16, 2, 4, 64, 2)
            : b >= 2 ? W4_DEC(1, 3, 12, 2, 4, 64, 3)
            : b == 1 ? W4_DEC(1, 1, 4, 2, 4, 64, 3)
                     : W4_DEC(1, 1, 4, 2, 4, 64, 2);
    }
#undef W4_DEC
    return hipGetLastError();
}

hipError_t launch_decode_int8(const void *x, int m, int64_t k, const void *packed,
                              const void *scales, int64_t n_out, const void *bias, void *y,
                              bool geglu, bool tiled, hipStream_t stream)
{
#define W8_LAYOUT(G, T) launch_decode_layout8<G, T>(x, m, k, packed, scales, n_out, bias, y, stream)
    if (geglu)
        return tiled ? W8_LAYOUT(true, true) : W8_LAYOUT(true, false);
    return tiled ? W8_LAYOUT(false, true) : W8_LAYOUT(false, false);
#undef W8_LAYOUT
}

}  // namespace w4a16
