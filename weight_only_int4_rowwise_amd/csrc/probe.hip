// HBM read probe: a measurement utility beside the method's kernels, not a
// step of it.  It reads a buffer once with the plainest streaming pattern,
// so the benchmark can set each decode launch next to what a bare stream of
// the same bytes costs on the same GPU: the read ceiling and the fixed cost
// of one launch (dispatch, first-load latency, the last wavefront's tail).
//
// One workgroup of 12 wavefronts per CU (256 x 768 threads); wavefront w of
// the grid reads the 1 KB blocks w, w + W, w + 2 W, ... (W = all
// wavefronts), four loads in flight each, so at any moment the whole chip
// reads one contiguous window of memory.  Nothing is computed but an xor of
// the data, which keeps the loads live; a lane whose xor hits a fixed
// constant stores it to the sink (practically never, and the same value
// whoever stores it).
#include "common.hpp"

namespace w4a16 {

constexpr int kProbeGroups = 256, kProbeThreads = 768, kProbeDepth = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src,
                                                                   int64_t blocks,
                                                                   uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x % kWave;
    const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / kWave);
    const int64_t w = (int64_t)blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t b = w;
    for (; b + (kProbeDepth - 1) * waves < blocks; b += kProbeDepth * waves) {
        u32x4 v[kProbeDepth];
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d)
            v[d] = __builtin_nontemporal_load(&src[(b + d * waves) * kWave + lane]);
#pragma unroll
        for (int d = 0; d < kProbeDepth; ++d)
            acc ^= v[d];
    }
    for (; b < blocks; b += waves)
        acc ^= __builtin_nontemporal_load(&src[b * kWave + lane]);
    const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == 0x9e3779b9u)
        *sink = r;
}

hipError_t launch_read_probe(const void *src, int64_t bytes, void *sink, hipStream_t stream)
{
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeGroups), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4 *>(src), bytes / 1024, static_cast<uint32_t *>(sink));
    return hipGetLastError();
}

}  // namespace w4a16
