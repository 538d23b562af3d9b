// Decode kernels of the zero-point INT4 variant: the INT4 launch table with
// the zero point subtracted in the dequantizer.
#include "decode.hpp"

namespace w4a16 {

hipError_t launch_decode_zp(const void *x, int m, int64_t k, const void *packed,
                            const void *scales, int64_t n_out, const void *bias, const void *zeros,
                            void *y, bool geglu, bool tiled, hipStream_t stream)
{
#define ZP_LAYOUT(G, T) launch_decode_layout4<G, T, true>(x, m, k, packed, scales, n_out, bias, zeros, y, stream)
    if (geglu)
        return tiled ? ZP_LAYOUT(true, true) : ZP_LAYOUT(true, false);
    return tiled ? ZP_LAYOUT(false, true) : ZP_LAYOUT(false, false);
#undef ZP_LAYOUT
}

}  // namespace w4a16
