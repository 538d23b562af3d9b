// Skinny W4A16 GEMM (16 < m <= 64) for gfx950.
//
// Same result definition as the decode and prefill kernels (GLM-130B paper
// card, "Method"; paperlayer.ai summary, "INT4 Quantization for RTX
// 3090s/2080s"): y[i][r] = fp16(s[r] * sum_c x[i][c] * q[r][c] + bias[r]),
// fp32 accumulation, optional fused GeGLU (paper card "Hyperparameters";
// paperlayer.ai B.3).
//
// Between decode and prefill the weight stream still dominates the bytes
// (k/2 per row against 2 m k for all activations), but every dequantized
// weight operand now feeds two to four MFMAs, so the kernel has to be an
// HBM stream and an MFMA pipeline at once.  Design:
//  * A workgroup owns G groups of 16 output rows and all B = ceil(m/16)
//    token blocks: T = G B output tiles of 16 x 16, cut into four equal
//    consecutive runs, one per wavefront (group-major order, so a wave
//    dequantizes at most ceil(T/4B) + 1 row groups per step).  G is chosen
//    per shape so that the grid covers the 256 compute units evenly (the
//    QKV projection has 2304 row groups = 9 per unit).
//  * Both operands reach LDS by LDS DMA (buffer loads written straight to
//    LDS), through a ring of S stages of 128 reduction indices: stage s
//    holds the 16 B x 128 activation tile and the R packed weight tiles (1 KB
//    each, the MFMA lane order of the prepacked layout).  Vector loads
//    retire in order, so the only way to keep many weight bytes in flight
//    behind the activation loads is to prefetch both S - 1 stages ahead.
//  * Every wave issues the same number of DMA loads per stage (the weight
//    slots are padded to a multiple of four; padding slots load zeros), so
//    one wait count, vmcnt(loads per stage x (S - 2)), says "stage s has
//    landed" for every wave; the barrier after it publishes the stage and
//    retires the slot the next DMA overwrites.
//  * Activation tiles are stored piece-major inside blocks of 16 tokens,
//    so an MFMA B-operand read is four contiguous 256-byte blocks (no bank
//    conflicts on gfx950).
//  * Steps past the end load zeros (out-of-range offsets), which keeps the
//    wait counts uniform; the loop drains all loads before the epilogue.
#include "common.hpp"

namespace w4a16 {

template <int B, int G, int S, int NWV, bool EVEN, bool GEGLU, bool TILED>
struct SkinnyShape {
    static constexpr int R = GEGLU ? 2 * G : G;          // weight row groups per workgroup
    static constexpr int XB = B * 4096;                  // activation bytes per stage
    static constexpr int SB = XB + R * 1024;             // stage bytes
    static constexpr int NX = 4 * B;                     // activation DMA loads per stage
    static constexpr int NITEM = NX + R;                 // DMA loads per stage (all waves)
    static constexpr int T = G * B;                      // output tiles per workgroup
    static constexpr int H = GEGLU ? 2 : 1;              // accumulators per tile
    static constexpr int NTHREADS = 64 * NWV;
    // DMA loads of wave w per stage: items w, w + NWV, ...
    static constexpr int items(int w) { return (NITEM - w + NWV - 1) / NWV; }
    static constexpr int MAXITEMS = items(0);
    // Tiles of wave w.  Waves w and w + 4 share a SIMD; each SIMD gets T/4
    // consecutive tiles (rounded), split between its waves.
    static constexpr int simd_t0(int s) { return s * T / 4; }
    static constexpr int tile0(int w)
    {
        return NWV == 4 ? simd_t0(w)
                        : (w < 4 ? simd_t0(w)
                                 : simd_t0(w - 4) + (simd_t0(w - 3) - simd_t0(w - 4) + 1) / 2);
    }
    static constexpr int tile1(int w)
    {
        return NWV == 4 ? simd_t0(w + 1)
                        : (w < 4 ? simd_t0(w) + (simd_t0(w + 1) - simd_t0(w) + 1) / 2
                                 : simd_t0(w - 3));
    }
    static constexpr int ntiles_max()
    {
        int mx = 0;
        for (int w = 0; w < NWV; ++w)
            mx = tile1(w) - tile0(w) > mx ? tile1(w) - tile0(w) : mx;
        return mx;
    }
    static constexpr int NTMAX = ntiles_max();
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    static_assert(S >= 2 && MAXITEMS * (S - 2) <= 63, "wait count out of range");
    static_assert(S * SB <= 160 * 1024, "LDS ring too large");
};

// Compute one stage for wave W: tiles [tile0(W), tile1(W)).
template <int W, int B, int G, int S, int NWV, bool EVEN, bool GEGLU, bool TILED>
__device__ __forceinline__ void skinny_compute(const uint8_t *stage, int lane,
                                               float4v (&acc)[SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>::NTMAX]
                                                             [SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>::H])
{
    using Sh = SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>;
    constexpr int t0 = Sh::tile0(W), t1 = Sh::tile1(W);
    if constexpr (t1 > t0) {
        constexpr int g0 = t0 / B, g1 = (t1 - 1) / B, NG = g1 - g0 + 1;
        const int r16 = lane % 16, g = lane / 16;
        // packed weights of this wave's row groups: one 16-byte read per group
        u32x4 wv[NG][Sh::H];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int h = 0; h < Sh::H; ++h)
                wv[q][h] = *reinterpret_cast<const u32x4 *>(stage + Sh::XB + (h * G + g0 + q) * 1024 + 16 * lane);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 a[NG][Sh::H];
#pragma unroll
            for (int q = 0; q < NG; ++q)
#pragma unroll
                for (int h = 0; h < Sh::H; ++h)
                    a[q][h] = dequant8_of<TILED>(wv[q][h][t]);
            half8 bx[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                bool used = false;
#pragma unroll
                for (int u = t0; u < t1; ++u)
                    used |= (u % B) == b;
                if (used)
                    bx[b] = as_half8(*reinterpret_cast<const u32x4 *>(
                        stage + ((16 * b + 4 * g + t) * 256) + 16 * r16));
            }
#pragma unroll
            for (int u = t0; u < t1; ++u)
#pragma unroll
                for (int h = 0; h < Sh::H; ++h)
                    acc[u - t0][h] = mfma16x16x32(a[u / B - g0][h], bx[u % B], acc[u - t0][h]);
        }
    }
}

// Per-lane load offsets of one wave: DMA item i of the wave is stage item
// w + NWV i; items below NX are activation chunks, the rest weight slots.
template <int B, int G, int S, int NWV, bool EVEN, bool GEGLU, bool TILED>
struct SkinnyLoads {
    using Sh = SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>;
    __amdgpu_buffer_rsrc_t wrs, xrs;
    uint32_t base[Sh::MAXITEMS], xcol[Sh::MAXITEMS];
    uint32_t k32;
    int64_t nsteps;
};

// Main loop and epilogue of wave W (a separate instantiation per wave, so
// each wave's accumulators keep fixed registers for the whole loop).
template <int W, int B, int G, int S, int NWV, bool EVEN, bool GEGLU, bool TILED>
__device__ __forceinline__ void skinny_wave(const SkinnyLoads<B, G, S, NWV, EVEN, GEGLU, TILED> &L,
                                            uint8_t *ring, int lane, int m, int64_t grp0,
                                            const uint16_t *__restrict__ scales, int64_t n_out,
                                            const uint16_t *__restrict__ bias,
                                            uint16_t *__restrict__ y)
{
    using Sh = SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>;
    constexpr int NI = Sh::items(W);
    constexpr int t0 = Sh::tile0(W), t1 = Sh::tile1(W);
    const int r16 = lane % 16;
    const int g = lane / 16;

    float4v acc[Sh::NTMAX][Sh::H];
#pragma unroll
    for (int u = 0; u < Sh::NTMAX; ++u)
#pragma unroll
        for (int h = 0; h < Sh::H; ++h)
            acc[u][h] = float4v{0.f, 0.f, 0.f, 0.f};

    // Offsets below 2^31 plus kOutOfRange stay below 2^32 and out of range.
    auto issue = [&](int64_t s) {
        uint8_t *st = ring + (s % S) * Sh::SB;
        const bool live = s < L.nsteps;
        const uint32_t xs = live ? (uint32_t)s * 256u : kOutOfRange;
        const uint32_t ws = live ? (TILED ? (uint32_t)s * 1024u : (uint32_t)s * 64u) : kOutOfRange;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int item = W + NWV * i;
            if (item < Sh::NX) {
                uint32_t off = L.base[i] + xs;
                if (!EVEN && (uint32_t)s * 128u + L.xcol[i] >= L.k32)
                    off = kOutOfRange;
                buf_load16_lds(L.xrs, off, st + 1024 * item);
            } else {
                uint32_t off = L.base[i] == kOutOfRange ? kOutOfRange : L.base[i] + ws;
                if (!EVEN && !TILED && (uint32_t)s * 128u + 32 * g >= L.k32)
                    off = kOutOfRange;
                buf_load16_lds(L.wrs, off, st + 1024 * item);
            }
        }
    };

#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        issue(s);
    for (int64_t s = 0; s < L.nsteps; ++s) {
        // this wave's loads of stage s have landed (S - 2 later stages may
        // be in flight); after the barrier every wave's have, and every
        // wave is done with stage s - 1, whose slot the next issue reuses
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI * (S - 2)));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        issue(s + S - 1);
        skinny_compute<W, B, G, S, NWV, EVEN, GEGLU, TILED>(ring + (s % S) * Sh::SB, lane, acc);
    }
    // the zero-filling loads past the end must land before the workgroup's
    // LDS can be handed to another workgroup
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // epilogue: tile t0 + u is output group (t0 + u) / B, token block
    // (t0 + u) % B; the lane holds outputs 4 g .. 4 g + 3 of the group for
    // token 16 b + r16
    const bool vec = (n_out % 4) == 0;
#pragma unroll
    for (int u = 0; u < t1 - t0; ++u) {
        const int tile = t0 + u;
        const int64_t mi = 16 * (tile % B) + r16;
        const int64_t ob = 16 * (grp0 + tile / B) + 4 * g;
        if (mi >= m || ob >= n_out)
            continue;
        uint16_t hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t o = ob + i < n_out ? ob + i : n_out - 1;
            float v;
            if (GEGLU) {
                float a = acc[u][0][i] * half_bits_to_float(scales[o]);
                float bv = acc[u][Sh::H - 1][i] * half_bits_to_float(scales[n_out + o]);
                if (bias) {
                    a += half_bits_to_float(bias[o]);
                    bv += half_bits_to_float(bias[n_out + o]);
                }
                v = gelu_erf(a) * bv;
            } else {
                v = acc[u][0][i] * half_bits_to_float(scales[o]);
                if (bias)
                    v += half_bits_to_float(bias[o]);
            }
            hv[i] = float_to_half_bits(v);
        }
        uint16_t *dst = y + mi * n_out + ob;
        if (vec && ob + 3 < n_out) {
            uint2 pk;
            pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
            pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
            *reinterpret_cast<uint2 *>(dst) = pk;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (ob + i < n_out)
                    dst[i] = hv[i];
        }
    }
}

template <int B, int G, int S, int NWV, bool EVEN, bool GEGLU, bool TILED>
__global__ __launch_bounds__(64 * NWV) void skinny_kernel(const uint16_t *__restrict__ x, int m,
                                                          int64_t k,
                                                          const uint8_t *__restrict__ packed,
                                                          const uint16_t *__restrict__ scales,
                                                          int64_t n_out,
                                                          const uint16_t *__restrict__ bias,
                                                          uint16_t *__restrict__ y)
{
    using Sh = SkinnyShape<B, G, S, NWV, EVEN, GEGLU, TILED>;
    using Ld = SkinnyLoads<B, G, S, NWV, EVEN, GEGLU, TILED>;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[S * Sh::SB];

    const int lane = threadIdx.x % kWave;
    // the wave index is uniform: keep it scalar so the per-wave dispatch
    // below is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane % 16;
    const int g = lane / 16;
    const int64_t grp0 = (int64_t)blockIdx.x * G;         // first output group
    const int64_t kb = k / 2;
    const int64_t kt = (k + 127) / 128;
    const int64_t rows = GEGLU ? 2 * n_out : n_out;
    const int64_t groups = (rows + 15) / 16;

    Ld L;
    L.wrs = make_rsrc(packed, weight_bytes(TILED, rows, k));
    L.xrs = make_rsrc(x, (int64_t)m * k * 2);
    L.k32 = (uint32_t)k;
    L.nsteps = kt;
#pragma unroll
    for (int i = 0; i < Sh::MAXITEMS; ++i) {
        const int item = wave + NWV * i;
        uint32_t off = kOutOfRange, col = 0;
        if (item < Sh::NX) {
            // activation chunk c = item: token block c / 4, pieces 4 (c % 4)
            // .. + 3; lane l fetches token 16 (c / 4) + l % 16 (tokens past
            // m repeat token m - 1), piece 4 (c % 4) + l / 16
            const int tok = 16 * (item / 4) + lane % 16;
            const int piece = 4 * (item % 4) + lane / 16;
            const int mi = tok < m ? tok : m - 1;
            col = 8 * piece;
            off = (uint32_t)(((int64_t)mi * k + 8 * piece) * 2);
        } else if (item < Sh::NITEM) {
            // weight slot r: output group grp0 + r (r < G); for GeGLU slot
            // G + j is the value group of output group grp0 + j
            const int r = item - Sh::NX;
            const int j = r < G ? r : r - G;
            const bool value = GEGLU && r >= G;
            if (TILED) {
                // prepacked GeGLU needs f % 16 == 0: value groups start at group f / 16
                const int64_t grp = (value ? n_out / 16 : 0) + grp0 + j;
                if (grp < groups)
                    off = (uint32_t)(grp * kt * 1024 + 16 * lane);
            } else {
                int64_t row = (value ? n_out : 0) + 16 * (grp0 + j) + r16;
                if (row >= rows)
                    row = rows - 1;           // outputs of clamped rows are never stored
                off = (uint32_t)(row * kb + 16 * g);
            }
        }
        L.base[i] = off;
        L.xcol[i] = col;
    }

#define W4_WAVE(W)                                                                                 \
    case W:                                                                                        \
        if constexpr (W < NWV)                                                                     \
            skinny_wave<W, B, G, S, NWV, EVEN, GEGLU, TILED>(L, ring, lane, m, grp0, scales, n_out, \
                                                             bias, y);                             \
        break;
    switch (wave) {
        W4_WAVE(0) W4_WAVE(1) W4_WAVE(2) W4_WAVE(3) W4_WAVE(4) W4_WAVE(5) W4_WAVE(6) W4_WAVE(7)
    }
#undef W4_WAVE
}

template <int B, int G, int S, int NWV, bool GEGLU, bool TILED>
hipError_t launch_skinny_t(const void *x, int m, int64_t k, const void *packed, const void *scales,
                           int64_t n_out, const void *bias, void *y, hipStream_t stream)
{
    const int64_t grid = ((n_out + 15) / 16 + G - 1) / G;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
#define W4_SKINNY(EV)                                                                              \
    hipLaunchKernelGGL((skinny_kernel<B, G, S, NWV, EV, GEGLU, TILED>), dim3((unsigned)grid),     \
                       dim3(64 * NWV), 0, stream, static_cast<const uint16_t *>(x), m, k,          \
                       static_cast<const uint8_t *>(packed), static_cast<const uint16_t *>(scales), \
                       n_out, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y))
    if (k % 128 == 0)
        W4_SKINNY(true);
    else
        W4_SKINNY(false);
#undef W4_SKINNY
    return hipGetLastError();
}

// Launch rules (measured on MI355X at the GLM-130B shapes).  The skinny
// kernel beats the decode kernel for 32 < m <= 64 on tall weights, where
// G output groups per workgroup put exactly one workgroup on each of the
// 256 compute units: the QKV projection (2304 groups, G = 9), the plain
// FFN up-projection (4096, G = 16) and the fused GeGLU up-projection (2048
// feature groups, G = 8).  Returns hipErrorNotSupported when no
// instantiation fits, and the caller uses the decode kernel.
template <bool GEGLU, bool TILED>
static hipError_t launch_skinny_layout(const void *x, int m, int64_t k, const void *packed,
                                       const void *scales, int64_t n_out, const void *bias,
                                       void *y, hipStream_t stream)
{
    const int64_t groups = (n_out + 15) / 16;
    if (m <= 32 || m > 64)
        return hipErrorNotSupported;
    const bool b3 = m <= 48;
    if constexpr (GEGLU) {
        if (groups == 8 * 256)
            return b3 ? launch_skinny_t<3, 8, 4, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream)
                      : launch_skinny_t<4, 8, 3, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
        return hipErrorNotSupported;
    } else {
        if (groups == 9 * 256)
            return b3 ? launch_skinny_t<3, 9, 5, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream)
                      : launch_skinny_t<4, 9, 3, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
        if (groups == 16 * 256)
            return b3 ? launch_skinny_t<3, 16, 4, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream)
                      : launch_skinny_t<4, 16, 4, 8, GEGLU, TILED>(x, m, k, packed, scales, n_out, bias, y, stream);
        return hipErrorNotSupported;
    }
}

hipError_t launch_skinny(const void *x, int m, int64_t k, const void *packed, const void *scales,
                         int64_t n_out, const void *bias, void *y, bool geglu, bool tiled,
                         hipStream_t stream)
{
    if (geglu)
        return tiled ? launch_skinny_layout<true, true>(x, m, k, packed, scales, n_out, bias, y, stream)
                     : launch_skinny_layout<true, false>(x, m, k, packed, scales, n_out, bias, y, stream);
    return tiled ? launch_skinny_layout<false, true>(x, m, k, packed, scales, n_out, bias, y, stream)
                 : launch_skinny_layout<false, false>(x, m, k, packed, scales, n_out, bias, y, stream);
}

}  // namespace w4a16
