/*
 * w8a16.h -- C ABI of the INT8 row-wise variant (W8A16) in the same
 * MI355X (gfx950) library as w4a16.h.
 *
 * The method is the one of w4a16.h with b = 8 bits per code: the paper card
 * (wikillm.com, "GLM-130B: An Open Bilingual Pre-trained Model"), section
 * "Paper vs code", bullet "Quantization scale", gives the scale of a b-bit
 * code as the row's absmax over 2^(b-1) - 1, which is 127 for b = 8; its
 * "Hyperparameters" table reports INT8 weights beside INT4 and FP16.  So
 *   s[r] = fp16(max_c |W[r][c]| / 127),  q = clamp(round(W / s), -127, 127)
 * and the linears multiply the FP16 activations by s * q.
 *
 * Every convention of w4a16.h holds (device pointers, 16-byte alignment,
 * stream semantics, ownership, error checks, the 2 GiB size limit, empty
 * calls, the status codes of w4a16_status and w4a16_last_error).  Codes are
 * stored one per byte as 8-bit two's complement, layout int8 [n][k] (the
 * pages fix no encoding; this is the plainest reading).
 */
#ifndef W8A16_H
#define W8A16_H

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * quantize_rowwise_int8 -- the quantizer with b = 8.
 *
 *   w_fp16      in   fp16  [n][k]  weight, out_features x in_features
 *   n, k             n >= 0, k >= 2, k even
 *   codes_i8    out  int8  [n][k]  codes in [-127, 127]
 *   scales_fp16 out  fp16  [n]     s[r] = fp16_rne(max_c |w[r][c]| / 127)
 *
 * Codes are round-half-to-even of the exact quotient w / s (against the
 * stored fp16 scale), clamped to [-127, 127]; a row whose scale rounds to
 * 0 gets s = 0 and all-zero codes.  Weights must be finite.  Deterministic.
 */
w4a16_status quantize_rowwise_int8(const void *w_fp16, int64_t n, int64_t k,
                                   void *codes_i8, void *scales_fp16, void *stream);

/*
 * w8a16_linear -- y[i][r] = fp16_rne( s[r] * sum_c x[i][c] * q[r][c] (+ bias[r]) ),
 * fp32 accumulation, the scale applied once per output after the sum.
 *
 *   x_fp16      in   fp16  [m][k]  m >= 0, k > 0, k % 32 == 0
 *   codes_i8    in   int8  [n][k]  from quantize_rowwise_int8
 *   scales_fp16 in   fp16  [n]
 *   bias_fp16   in   fp16  [n] or NULL
 *   y_fp16      out  fp16  [m][n]
 *
 * Kernel choice by m as in w4a16_linear.  Deterministic.
 */
w4a16_status w8a16_linear(const void *x_fp16, int64_t m, int64_t k,
                          const void *codes_i8, const void *scales_fp16, int64_t n,
                          const void *bias_fp16, void *y_fp16, void *stream);

/*
 * w8a16_geglu_linear -- the fused GeGLU up-projection of w4a16_geglu_linear
 * over INT8 codes [2f][k] (rows [0, f) gated by GELU, rows [f, 2f) linear),
 * output fp16 [m][f].
 */
w4a16_status w8a16_geglu_linear(const void *x_fp16, int64_t m, int64_t k,
                                const void *codes_i8, const void *scales_fp16, int64_t f,
                                const void *bias_fp16, void *y_fp16, void *stream);

/*
 * Prepacked INT8 layout: the load-time tile order of w4a16.h's prepacked
 * layout with one byte per code.  Tile (g, t) -- rows [16g, 16g+16),
 * features [128t, 128t+128) -- is 2048 bytes at ((g * ceil(k/128)) + t) *
 * 2048; byte h * 1024 + 16 * l + e (h < 2, l = 16 j + r, j < 4, r < 16,
 * e < 16) holds the code of row 16g + r, feature 128t + 32j + 16h + e, as
 * the offset byte q + 128 (q's two's complement with the top bit flipped).
 * Rows past n and features past k hold code 0 (byte 0x80).
 *
 * w8a16_prepacked_bytes: ceil(n/16) * ceil(k/128) * 2048, or -1 if n < 0,
 *   k <= 0 or k % 32 != 0.
 * w8a16_prepack: codes_i8 [n][k] -> codes_prepacked (w8a16_prepacked_bytes
 *   bytes), k % 32 == 0.
 * w8a16_linear_prepacked / w8a16_geglu_linear_prepacked: the linears on the
 *   prepacked layout (n = number of rows, or 2f with f % 16 == 0 for
 *   GeGLU); the results are bit-identical to the row-major calls.
 */
int64_t w8a16_prepacked_bytes(int64_t n, int64_t k);

w4a16_status w8a16_prepack(const void *codes_i8, int64_t n, int64_t k, void *codes_prepacked,
                           void *stream);

w4a16_status w8a16_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                    const void *codes_prepacked, const void *scales_fp16,
                                    int64_t n, const void *bias_fp16, void *y_fp16,
                                    void *stream);

w4a16_status w8a16_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                          const void *codes_prepacked, const void *scales_fp16,
                                          int64_t f, const void *bias_fp16, void *y_fp16,
                                          void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A16_H */
