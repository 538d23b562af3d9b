// Load-time weight layout transform (the pages' FasterTransformer port
// "pre-transposes parameters": paperlayer.ai summary, section B.5).
//
// Row-major packed codes [n][k/2] -> prepacked tiles.  Tile (g, t) covers
// weight rows [16 g, 16 g + 16) and reduction indices [128 t, 128 t + 128):
// 1024 bytes, stored at ((g * ceil(k/128)) + t) * 1024, laid out in the
// order the MFMA A operand is loaded: 16 bytes per lane, lane l = 16 j + r
// holding row 16 g + r, packed bytes [64 t + 16 j, +16) of that row, with
// the nibbles of each dword reordered for dequant8 (codes e0..e7 of the
// dword as bytes e0|e2<<4, e4|e6<<4, e1|e3<<4, e5|e7<<4).  Rows past n and
// indices past k are zero codes.  Same codes, same two's-complement nibble
// encoding: only their order changes, so every 1 KB tile is one contiguous
// read for a wavefront.
#include "common.hpp"

namespace w4a16 {

__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t *__restrict__ src, int64_t n,
                                                      int64_t k, uint8_t *__restrict__ dst,
                                                      int64_t total_pieces)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total_pieces)
        return;
    const int64_t kt = (k + 127) / 128;
    const int lane = (int)(idx % 64);
    const int64_t tile = idx / 64;
    const int64_t grp = tile / kt;
    const int64_t t = tile % kt;
    const int64_t row = 16 * grp + lane % 16;
    const int64_t byte = 64 * t + 16 * (lane / 16);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < n && byte < k / 2) {
        v = load16(src + row * (k / 2) + byte);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = prepack_nibbles(v[i]);
    }
    *reinterpret_cast<u32x4 *>(dst + idx * 16) = v;
}

// INT8 codes [n][k] -> prepacked tiles of 16 rows x 128 indices, 2 KB each,
// stored at ((g * ceil(k/128)) + t) * 2048: two 1 KB halves in lane order,
// lane l = 16 j + r holding row 16 g + r, codes [128 t + 32 j + 16 h, +16)
// in half h, natural order, each as the offset byte q + 128 (the two's
// complement with its top bit flipped) that dequant8_i8 reads.  Rows past
// n and indices past k hold code 0 (byte 0x80).
__global__ __launch_bounds__(256) void prepack8_kernel(const uint8_t *__restrict__ src, int64_t n,
                                                       int64_t k, uint8_t *__restrict__ dst,
                                                       int64_t total_pieces)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total_pieces)
        return;
    const int64_t kt = (k + 127) / 128;
    const int lane = (int)(idx % 64);
    const int h = (int)((idx / 64) % 2);
    const int64_t tile = idx / 128;
    const int64_t grp = tile / kt;
    const int64_t t = tile % kt;
    const int64_t row = 16 * grp + lane % 16;
    const int64_t col = 128 * t + 32 * (lane / 16) + 16 * h;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < n && col < k)
        v = load16(src + row * k + col);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] ^= 0x80808080u;
    *reinterpret_cast<u32x4 *>(dst + idx * 16) = v;
}

int64_t prepacked_bytes_int8(int64_t n, int64_t k)
{
    return ((n + 15) / 16) * ((k + 127) / 128) * 2048;
}

hipError_t launch_prepack_int8(const void *src, int64_t n, int64_t k, void *dst, hipStream_t stream)
{
    const int64_t pieces = prepacked_bytes_int8(n, k) / 16;
    const int64_t blocks = (pieces + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prepack8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(src), n, k, static_cast<uint8_t *>(dst), pieces);
    return hipGetLastError();
}

int64_t prepacked_bytes(int64_t n, int64_t k)
{
    return ((n + 15) / 16) * ((k + 127) / 128) * 1024;
}

hipError_t launch_prepack(const void *src, int64_t n, int64_t k, void *dst, hipStream_t stream)
{
    const int64_t pieces = prepacked_bytes(n, k) / 16;
    const int64_t blocks = (pieces + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(src), n, k, static_cast<uint8_t *>(dst), pieces);
    return hipGetLastError();
}

}  // namespace w4a16
