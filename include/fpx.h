/*
 * fpx.h -- C ABI of the same fused weight-only linear layer for float weights
 * of other bit widths: FP6 e2m3, FP5 e2m2 and FP4 e2m1 next to FP6 e3m2.
 *
 *   Y[M,N] = X[M,K] . dequant(W_fpx[N,K])^T,  X and Y fp16, one fp16 scale
 *   per output row, Wdq[n,k] = fp16_RNE(v(c[n,k]) * s_n), fp32 accumulation.
 *
 * FP6-LLM (arXiv 2401.14112), abstract: one full-stack kernel scheme with
 * Tensor-Core support for float weights of several quantisation bit widths.
 * TC-FPx explainer (duicuo.cn), section "redesigning the kernel solution": a
 * unified kernel for quantised weights of different widths up to 6 bits.  The
 * pages name no formats; these are the plainest IEEE-like ones (sign on top,
 * exponent bias 2^(E-1)-1, subnormals, no inf/NaN):
 *
 *   format  id  bits  bias  max   packed bytes  scale range accepted
 *   e3m2    0   6     3     28    0.75*N*K      finite, |s| < 16
 *   e2m3    1   6     1     7.5   0.75*N*K      finite, |s| < 4
 *   e2m2    2   5     1     7     0.625*N*K     finite, |s| < 4
 *   e2m1    3   4     1     6     0.5*N*K       finite
 *
 * (e3m2, e2m3 and e2m1 are the OCP MX v1.0 FP6 E3M2, FP6 E2M3 and FP4 E2M1
 * element formats.)  A code is an integer in [0, 2^bits): the sign is bit
 * bits-1, then the exponent, then the mantissa.  The scale range is where the
 * fused kernel's one fp16 multiply is exact (e3m2: s*2^12, e2m3 and e2m2:
 * s*2^14 must be fp16 numbers).
 *
 * Every format uses the conventions, size limits, status codes, plan
 * variants, split-K workspace and determinism of fp6.h; fpx_* with format 0
 * is the same as the matching fp6_* call.  An unknown format gives
 * FP6_E_VALUE (before any HIP call).
 *
 * Packed layout v3 for each format: tiles of 16 rows x 256 k at
 * (kb*(N/16) + nb) * tile_bytes (k-block major), tile_bytes = 4096*bits/8;
 * local row r, local k = 32*j + 8*g + i belong to wave lane L = 16*g + r.
 *   e3m2: as described in fp6.h.
 *   e2m3: planes placed as e3m2's, with 2-bit piece (s, e1) = c >> 4 and
 *         4-bit piece (e0 m2 m1 m0) = c & 15; in the 2-bit plane, with
 *         p = 4*(j%2) + i/2, h = i%2 and b = [0,1,2,3,8,9,10,11][p], bit e1
 *         is at b + 16h and bit s at b + 4 + 16h of word j/2 of lane L; in
 *         the 4-bit word j%4 element i is the nibble at slot i/2 + 4*(i%2).
 *   e2m2: 4-bit plane (e1 e0 m1 m0 = c & 15) at tile bytes [0,2048) laid out
 *         like the e3m2 one ([0,1024) k-steps 0..3, [1024,2048) k-steps 4..7,
 *         16 bytes per lane, word j%4, nibble slot 2*(i%4) + i/4); 1-bit
 *         plane (s = c >> 4) at [2048,2560): lane L's 8 bytes at 2048 + 8L,
 *         word j/4, bit (7 + 8*(i%4) + 2*(j%4) + i/4) mod 32 (layout v3;
 *         v1 and v2 had bit 4*(j%4) + i/2 + 16*(i%2), nibble slot
 *         i/2 + 4*(i%2)).
 *   e2m1: one 4-bit plane at [0,2048) laid out like the FP6 one but holding
 *         the whole code, element i in nibble slot i.
 */
#ifndef FPX_AMD_H
#define FPX_AMD_H

#include <stddef.h>
#include <stdint.h>

#include "fp6.h"

#ifdef __cplusplus
extern "C" {
#endif

enum fpx_format { FPX_E3M2 = 0, FPX_E2M3 = 1, FPX_E2M2 = 2, FPX_E2M1 = 3 };

/* Code width of a format (6, 6, 5, 4), or 0 for an unknown format. */
int fpx_bits(int format);

/* Bytes of the packed buffer: N*K*bits/8, or 0 for an unknown format or an
 * (N, K) outside the limits of fp6.h. */
size_t fpx_packed_bytes(int format, int64_t N, int64_t K);

/*
 * fpx_quantize_rows -- host, synchronous, deterministic; fp6_quantize_rows
 * for any format: s_n = fp16_RNE(max_k |W[n,k]| / max) and c = sign(W) on the
 * top bit | nearest magnitude index of |W / s_n| (double quotient, ties to the
 * even code, saturating at max; rows with s_n == 0 get all-zero codes).
 * Errors: FP6_E_NULL, FP6_E_SHAPE, FP6_E_VALUE (non-finite W or unknown
 * format), FP6_E_SCALE (a row scale outside the format's range).
 */
int fpx_quantize_rows(int format, const float* W, int64_t N, int64_t K, uint8_t* codes,
                      uint16_t* scales);

/*
 * fpx_prepack -- host, synchronous, pure (offline step): codes (host uint8
 * [N][K], each < 2^bits) into packed layout v3 of the format.  scales are
 * only checked against the format's range.  packed_bytes must equal
 * fpx_packed_bytes(format, N, K).  Errors: FP6_E_NULL, FP6_E_SHAPE,
 * FP6_E_CODE, FP6_E_SCALE, FP6_E_SIZE, FP6_E_VALUE (unknown format).
 */
int fpx_prepack(int format, const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                void* packed, size_t packed_bytes);

/*
 * fpx_linear / fpx_linear_plan -- device, asynchronous on `stream`: the fused
 * layer of fp6_linear / fp6_linear_plan for a packed weight of `format`
 * (same arguments, alignment, variants, splits and errors).
 */
int fpx_linear(int format, const void* X, const void* packed_W, const void* scales, void* Y,
               int64_t M, int64_t N, int64_t K, void* stream);
int fpx_linear_plan(int format, const void* X, const void* packed_W, const void* scales, void* Y,
                    int64_t M, int64_t N, int64_t K, int variant, int splits, void* stream);

/* fpx_dequant -- device, asynchronous; fp6_dequant for any format (the same
 * device splice-and-scale code as fpx_linear). */
int fpx_dequant(int format, const void* packed_W, const void* scales, void* W16, int64_t N,
                int64_t K, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FPX_AMD_H */
