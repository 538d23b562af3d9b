/*
 * w4a16_zp.h -- C ABI of the zero-point INT4 variant in the same MI355X
 * (gfx950) library as w4a16.h.
 *
 * The paper card (wikillm.com, "GLM-130B: An Open Bilingual Pre-trained
 * Model"), section "Pitfalls", reports a zero-point INT4 variant (LAMBADA
 * 80.63% against 79.47% for the row-wise absmax scheme) and notes that
 * absmax was chosen as the cheaper one; the pages give no formula.  This is
 * the standard asymmetric 4-bit quantizer, per output row r:
 *   lo = min(min_c W[r][c], 0),  hi = max(max_c W[r][c], 0)
 *   s[r] = fp16_rne((hi - lo) / 15)
 *   z[r] = clamp(round_half_even(-lo / s[r]), 0, 15)          (uint8)
 *   q[r][c] = clamp(round_half_even(W[r][c] / s[r]) + z[r], 0, 15)
 *   W_hat = s * (q - z)
 * with exact quotients; a row whose scale rounds to 0 gets z = 0 and all-zero
 * codes.  The range is widened to hold 0 so that the zero point is an
 * integer in [0, 15] and a zero weight decodes to exactly 0.
 *
 * Every convention of w4a16.h holds (device pointers, 16-byte alignment of
 * every pointer including zeros_u8, stream semantics, ownership, error
 * checks, size limits, empty calls, the status codes).  Codes are packed as
 * the INT4 ones (code 2j in the low nibble of byte j, 2j + 1 in the high
 * nibble), as unsigned 4-bit values; the zero points are uint8 [n].  The
 * prepacked layout is w4a16_prepack's (the same nibble reorder): use
 * w4a16_prepacked_bytes / w4a16_prepack on these codes too.
 */
#ifndef W4A16_ZP_H
#define W4A16_ZP_H

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * quantize_rowwise_int4_zp -- the quantizer above.
 *
 *   w_fp16      in   fp16  [n][k]    n >= 0, k >= 2, k even
 *   q_packed    out  uint8 [n][k/2]  unsigned codes, two per byte
 *   scales_fp16 out  fp16  [n]
 *   zeros_u8    out  uint8 [n]       zero points in [0, 15]
 * Weights must be finite.  Deterministic.
 */
w4a16_status quantize_rowwise_int4_zp(const void *w_fp16, int64_t n, int64_t k,
                                      void *q_packed, void *scales_fp16, void *zeros_u8,
                                      void *stream);

/*
 * w4a16_zp_linear -- y[i][r] = fp16_rne( s[r] * sum_c x[i][c] * (q[r][c] - z[r]) (+ bias[r]) ),
 * fp32 accumulation (the dequantized q - z are exact fp16 integers), the
 * scale applied once per output after the sum.
 *
 *   x_fp16 [m][k] (k % 32 == 0), q_packed [n][k/2], scales_fp16 [n],
 *   zeros_u8 [n], bias_fp16 [n] or NULL, y_fp16 [m][n].
 * Kernel choice by m as in w4a16_linear.  Deterministic.
 */
w4a16_status w4a16_zp_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                             const void *scales_fp16, const void *zeros_u8, int64_t n,
                             const void *bias_fp16, void *y_fp16, void *stream);

/* The fused GeGLU up-projection of w4a16_geglu_linear over zero-point codes
 * [2f][k/2] with scales and zero points [2f]; output fp16 [m][f]. */
w4a16_status w4a16_zp_geglu_linear(const void *x_fp16, int64_t m, int64_t k, const void *q_packed,
                                   const void *scales_fp16, const void *zeros_u8, int64_t f,
                                   const void *bias_fp16, void *y_fp16, void *stream);

/* The two linears on codes reordered by w4a16_prepack (f % 16 == 0 for
 * GeGLU); bit-identical to the row-major calls. */
w4a16_status w4a16_zp_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                       const void *q_prepacked, const void *scales_fp16,
                                       const void *zeros_u8, int64_t n, const void *bias_fp16,
                                       void *y_fp16, void *stream);

w4a16_status w4a16_zp_geglu_linear_prepacked(const void *x_fp16, int64_t m, int64_t k,
                                             const void *q_prepacked, const void *scales_fp16,
                                             const void *zeros_u8, int64_t f,
                                             const void *bias_fp16, void *y_fp16, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_ZP_H */
