// Decode kernels of the INT4 path (the launch table is in decode.hpp), and
// the decode entry that picks the code kind: INT4, its zero-point variant
// (decode_zp.hip) or INT8 (decode_w8.hip), each compiled on its own.
#include "decode.hpp"

namespace w4a16 {

hipError_t launch_decode_int8(const void *x, int m, int64_t k, const void *packed,
                              const void *scales, int64_t n_out, const void *bias, void *y,
                              bool geglu, bool tiled, hipStream_t stream);
hipError_t launch_decode_zp(const void *x, int m, int64_t k, const void *packed,
                            const void *scales, int64_t n_out, const void *bias, const void *zeros,
                            void *y, bool geglu, bool tiled, hipStream_t stream);

hipError_t launch_decode(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, const void *zeros, void *y, bool geglu,
                         bool tiled, int cb, hipStream_t stream)
{
    if (cb == 8)
        return launch_decode_int8(x, m, k, packed, scales, n_out, bias, y, geglu, tiled, stream);
    if (zeros)
        return launch_decode_zp(x, m, k, packed, scales, n_out, bias, zeros, y, geglu, tiled, stream);
#define W4_LAYOUT(G, T) launch_decode_layout4<G, T, false>(x, m, k, packed, scales, n_out, bias, nullptr, y, stream)
    if (geglu)
        return tiled ? W4_LAYOUT(true, true) : W4_LAYOUT(true, false);
    return tiled ? W4_LAYOUT(false, true) : W4_LAYOUT(false, false);
#undef W4_LAYOUT
}

}  // namespace w4a16
