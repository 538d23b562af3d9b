/*
 * w4a16.h -- C ABI of the MI355X (gfx950) weight-only INT4 row-wise library.
 *
 * The method (GLM-130B, "GLM-130B: An Open Bilingual Pre-trained Model"):
 * every FP16 weight matrix of a linear layer, laid out [out_features][in_features],
 * is quantized with one absmax scale per output row, s = fp16(max|W[n,:]| / 7),
 * to integer codes q = clamp(round(W / s), -7, 7) packed two per byte; at run
 * time the FP16 activations multiply the dequantized weights s * q.
 *   - wikillm.com paper card, section "Method": weight-only INT4 paragraph and
 *     the quantize_linear_int4 / linear_forward pseudocode;
 *   - same card, section "Paper vs code", bullet "Quantization scale": divisor
 *     2^(b-1) - 1 = 7, computed per output row in FP16, then rounding and
 *     int8 packing; bullet "Quantized layers": QKV, attention output and both
 *     MLP projections are quantized, biases stay FP16;
 *   - same card, "Hyperparameters": hidden 12288, FFN 32768 (GeGLU);
 *   - paperlayer.ai summary, "INT4 Quantization for RTX 3090s/2080s": FP16
 *     activations, weights turned back into FP16 at run time.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory),
 *    row-major and contiguous, and must be 16-byte aligned.
 *  - fp16 means IEEE binary16.  Packed weights are uint8 [n][k/2]: code
 *    q[n][2j] is the low nibble and q[n][2j+1] the high nibble of byte
 *    [n][j], each as 4-bit two's complement (the pages fix neither order nor
 *    encoding; this is the plainest reading).  Codes are in [-7, 7].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work: they return before the GPU finishes, and a fault inside a
 *    kernel surfaces at the caller's next synchronisation.
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    device or host memory, keeps no pointer after returning, and has no
 *    mutable global state apart from a per-thread last-error string: calls
 *    are reentrant and thread-safe.
 *  - Errors: every argument is checked before any HIP call; on a failed
 *    check nothing is enqueued and no memory is touched.  After the launch
 *    hipGetLastError() is read; a launch failure returns W4A16_ERR_HIP and
 *    w4a16_last_error() (per thread) names the HIP error.
 *  - Outputs must not overlap inputs.  Sizes are element counts.
 *  - Sizes are checked first.  m == 0 or n == 0 (f == 0) is then a valid
 *    empty call: nothing is launched and the pointers are not looked at
 *    (they may be NULL).
 *  - Size limit of the linears: the activations (2 m k bytes) and the
 *    packed weight (in its layout) must each be smaller than 2 GiB, since
 *    the kernels address them with 32-bit buffer offsets; larger calls
 *    return W4A16_ERR_SHAPE.  The largest GLM-130B weight (the 65536 x
 *    12288 GeGLU up-projection, 384 MiB packed) is far below it.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,   /* a required pointer is NULL */
    W4A16_ERR_SHAPE = 2,  /* a size is negative, k is 0, k violates the
                             divisibility rule of the call, or a size is too large */
    W4A16_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned */
    W4A16_ERR_HIP = 4,    /* the HIP runtime reported an error (see w4a16_last_error) */
    W4A16_ERR_DEVICE = 5  /* no code object for the current device (it is not gfx950) */
} w4a16_status;

#define W4A16_ABI_VERSION 1

/*
 * quantize_rowwise_int4 -- quantize_linear_int4 of the paper card ("Method").
 *
 *   w_fp16      in   fp16  [n][k]    weight, out_features x in_features
 *   n, k             n >= 0, k >= 2, k even
 *   q_packed    out  uint8 [n][k/2]  packed codes (layout above)
 *   scales_fp16 out  fp16  [n]       s[r] = fp16_rne(max_c |w[r][c]| / 7)
 *
 * Codes are round-half-to-even of the exact quotient w / s (against the
 * STORED fp16 scale), clamped to [-7, 7]; a row whose scale rounds to 0
 * (all-zero rows, or absmax <= 3 * 2^-24) gets s = 0 and all-zero codes.
 * Weights must be finite; for NaN or Inf inputs the outputs are unspecified.
 * The result is bit-for-bit deterministic.
 */
w4a16_status quantize_rowwise_int4(const void *w_fp16, int64_t n, int64_t k,
                                   void *q_packed, void *scales_fp16, void *stream);

/*
 * w4a16_linear -- linear_forward of the paper card ("Method"), W4A16:
 *   y[i][r] = fp16_rne( s[r] * sum_c x[i][c] * q[r][c]  (+ bias[r]) )
 * accumulated in fp32; the scale is applied once per output after the sum
 * (it is constant along the reduced dimension), the bias (if any) is added
 * in fp32, and there is one rounding to fp16.
 *
 *   x_fp16      in   fp16  [m][k]    activations (tokens x in_features)
 *   m, k             m >= 0, k > 0, k % 32 == 0
 *   q_packed    in   uint8 [n][k/2]  from quantize_rowwise_int4
 *   scales_fp16 in   fp16  [n]
 *   n                n >= 0
 *   bias_fp16   in   fp16  [n] or NULL
 *   y_fp16      out  fp16  [m][n]
 *
 * m <= 64 runs the memory-bound decode kernel, 64 < m <= 128 runs it twice
 * (tokens 0..63, then the rest), larger m runs the MFMA GEMM.  INT4 calls
 * also take the GEMM from a threshold between m = 65 and 120 where one GEMM
 * launch is faster than two decode launches; it depends on the weight's
 * rows (n, or 2f for GeGLU) and, for 8192 to 16383 plain rows, on k.  Plain
 * weights of fewer than 8192 rows take it only with k >= 8192 (from
 * m = 104), GeGLU weights of fewer than 12288 rows never.
 * Results are deterministic (no atomics, fixed reduction order).
 */
w4a16_status w4a16_linear(const void *x_fp16, int64_t m, int64_t k,
                          const void *q_packed, const void *scales_fp16, int64_t n,
                          const void *bias_fp16, void *y_fp16, void *stream);

/*
 * w4a16_geglu_linear -- the GeGLU up-projection of the FFN (paper card,
 * "Method" and "Hyperparameters"; paperlayer.ai summary, section B.3) fused
 * into the W4A16 linear:
 *   a[i][j] = linear through weight rows j        (j in [0, f))
 *   b[i][j] = linear through weight rows f + j
 *   y[i][j] = fp16_rne( GELU(a) * b ),  GELU(t) = t * Phi(t) (erf form)
 * where a and b are kept in fp32 (scale and bias applied) until the single
 * final rounding.  The pages do not say which half is gated; the first f
 * rows are taken as the GELU branch.
 *
 *   x_fp16      in   fp16  [m][k]      m >= 0, k > 0, k % 32 == 0
 *   q_packed    in   uint8 [2f][k/2]
 *   scales_fp16 in   fp16  [2f]
 *   f                f >= 0 (output width)
 *   bias_fp16   in   fp16  [2f] or NULL
 *   y_fp16      out  fp16  [m][f]
 */
w4a16_status w4a16_geglu_linear(const void *x_fp16, int64_t m, int64_t k,
                                const void *q_packed, const void *scales_fp16, int64_t f,
                                const void *bias_fp16, void *y_fp16, void *stream);

/*
 * Prepacked layout -- the load-time weight layout transform that the
 * pages' FasterTransformer port applies ("pre-transposing parameters",
 * paperlayer.ai summary, section B.5), here for gfx950's matrix cores.
 *
 * Same codes and nibble encoding as quantize_rowwise_int4's output, in
 * another order: the weight is cut into tiles of 16 rows x 128 input
 * features (1024 bytes); tile (g, t) -- rows [16g, 16g+16), features
 * [128t, 128t+128) -- is stored at byte ((g * ceil(k/128)) + t) * 1024, and
 * inside it the 16 bytes at offset 16 * l (l = 16 j + r, j < 4, r < 16) hold
 * packed bytes [64t + 16j, 64t + 16j + 16) of row 16g + r, with the codes
 * e0..e7 of each 4-byte word stored as the bytes e0|e2<<4, e4|e6<<4,
 * e1|e3<<4, e5|e7<<4 (the order the dequantizer unpacks).  Rows past n and
 * features past k are zero codes.  Each tile is then one contiguous read
 * in exactly the order the kernels consume it.
 *
 * w4a16_prepacked_bytes: size of the prepacked buffer,
 *   ceil(n/16) * ceil(k/128) * 1024, or -1 if n < 0, k <= 0 or k % 32 != 0.
 * w4a16_prepack: q_packed [n][k/2] (device) -> q_prepacked (device,
 *   w4a16_prepacked_bytes(n, k) bytes).  k % 32 == 0.  The reorder moves
 *   nibbles without reading them, so it serves the unsigned codes of the
 *   zero-point variant (w4a16_zp.h) as well.
 * w4a16_linear_prepacked / w4a16_geglu_linear_prepacked: exactly
 *   w4a16_linear / w4a16_geglu_linear with the weight in the prepacked
 *   layout; the GeGLU form needs f % 16 == 0 (the gate / value boundary
 *   falls on a tile boundary).  Results are bit-identical to the row-major
 *   calls for the same m (same kernels, same summation order).
 */
int64_t w4a16_prepacked_bytes(int64_t n, int64_t k);

w4a16_status w4a16_prepack(const void *q_packed, int64_t n, int64_t k, void *q_prepacked,
                           void *stream);

w4a16_status w4a16_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                    const void *q_prepacked, const void *scales_fp16, int64_t n,
                                    const void *bias_fp16, void *y_fp16, void *stream);

w4a16_status w4a16_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                          const void *q_prepacked, const void *scales_fp16,
                                          int64_t f, const void *bias_fp16, void *y_fp16,
                                          void *stream);

/* Measurement utility, not a step of the method: reads `bytes` of device
 * memory at `src` once (a multiple of 1024, 16-byte aligned, up to 2^40)
 * in the plainest streaming pattern (one 768-thread workgroup per CU, each
 * wavefront reading every W-th 1 KB block, W = all wavefronts, four loads
 * in flight), so that a decode launch can be set beside what a bare stream
 * of the same bytes costs on the same GPU.  `sink_u32` (4 bytes of device
 * memory, 4-byte aligned) may receive one word; its content is meaningless.
 * Stream-ordered on `stream`; allocates nothing.  Errors: W4A16_ERR_SHAPE,
 * W4A16_ERR_NULL, W4A16_ERR_ALIGN, W4A16_ERR_HIP. */
w4a16_status w4a16_read_probe(const void *src, int64_t bytes, void *sink_u32, void *stream);

/* Static English text for a status code (never NULL). */
const char *w4a16_status_string(int status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char *w4a16_last_error(void);

/* W4A16_ABI_VERSION of the built library. */
int w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
