/*
 * fp6s.h -- C ABI of the 2:4-sparse FP6 (e3m2) weight-only linear layer on
 * gfx950 sparse matrix cores (v_smfmac_f32_16x16x64_f16).
 *
 *   Y[M,N] = X[M,K] . Wdq^T,  Wdq[n,k] = fp16_RNE(v(c) * s_n) at kept
 *   positions and 0 elsewhere; in every aligned group of 4 weights along k at
 *   most 2 are kept.
 *
 * Sparse-Marlin (first page, post on quantised-weight kernels, points on 2:4
 * sparsity): quantised weights that are also 2:4 structured-sparse, run on
 * sparse matrix units, with the quantised values, the sparsity metadata and
 * the quantisation scales laid out together.  This is that idea for FP6 on
 * MI355X: the kept codes use the FP6 splice of fp6.h and the positions feed
 * the sparse MFMA's index operand directly.  Weight bytes: 0.5 per dense
 * weight (6-bit codes + 2-bit positions for half of them), 2/3 of dense FP6.
 *
 * Conventions, status codes, X / Y / scales layouts and alignment are those
 * of fp6.h.  Shapes: N % 16 == 0, K % 512 == 0 (other limits as fp6.h).
 *
 * Compressed form (host): codes uint8 [N][K/2] and pos uint8 [N][K/2]; entry
 * 2t+s of a row is the s-th kept weight (s = 0, 1) of the dense group t
 * (k = 4t..4t+3): its e3m2 code and its position 0..3 in the group, with
 * pos[2t] < pos[2t+1].  A kept weight may be zero.
 *
 * Packed 2:4 layout: tiles of 16 rows x 512 dense k (4096 bytes) at
 * (nb*(K/512) + kb)*4096.  For k-step j (64 dense k, one sparse MFMA) and wave
 * lane L = 16g + r (row r), element i (0..7) is kept weight i%2 of the dense
 * group at tile offset 64j + 32(g%2) + 16(i/4) + 8(g/2) + 4((i%4)/2).  Bytes
 * [0, 3072) hold the codes exactly where the dense layout (fp6.h) puts lane
 * L, k-step j, element i of an FP6 tile; bytes [3072, 4096) hold the
 * positions: lane L's 16 bytes at 3072 + 16L, word j/2, bits 16(j%2) + 2i.
 */
#ifndef FP6S_AMD_H
#define FP6S_AMD_H

#include <stddef.h>
#include <stdint.h>

#include "fp6.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the packed 2:4 buffer: N*K/2, or 0 if (N, K) is unsupported. */
size_t fp6s_packed_bytes(int64_t N, int64_t K);

/*
 * fp6s_prune_quantize -- host, synchronous, deterministic (input preparation;
 * the pages give no pruning rule).  In every group of 4 weights along k keeps
 * the 2 of largest magnitude (the lower index first among equal magnitudes),
 * then quantises the kept values per row as fp6_quantize_rows does
 * (s_n = fp16_RNE(max|kept| / 28)).  W: host float32 [N][K], finite, K % 4 ==
 * 0.  Outputs: codes, pos [N][K/2] (see above), scales fp16 bits [N].
 * Errors: FP6_E_NULL, FP6_E_SHAPE, FP6_E_VALUE (non-finite W), FP6_E_SCALE.
 */
int fp6s_prune_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes, uint8_t* pos,
                        uint16_t* scales);

/*
 * fp6s_prepack -- host, synchronous, pure: compressed form -> packed 2:4
 * layout.  packed_bytes must equal fp6s_packed_bytes(N, K).  Errors:
 * FP6_E_NULL, FP6_E_SHAPE, FP6_E_CODE (a code > 63), FP6_E_VALUE (positions
 * not increasing or > 3), FP6_E_SCALE (as fp6_prepack), FP6_E_SIZE.
 */
int fp6s_prepack(const uint8_t* codes, const uint8_t* pos, const uint16_t* scales, int64_t N,
                 int64_t K, void* packed, size_t packed_bytes);

/*
 * fp6s_linear -- device, asynchronous on `stream`: the fused 2:4-sparse layer
 * (de-quantise the kept codes in registers, sparse fp16 MFMA with fp32
 * accumulation, one final rounding to fp16).  Arguments and errors as
 * fp6_linear; the split-K workspace is shared with it.  Bitwise deterministic.
 */
int fp6s_linear(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                int64_t N, int64_t K, void* stream);

/*
 * fp6s_linear_plan -- fp6s_linear with the schedule forced.  variant:
 * 0 = automatic; 1 = k-slice (one workgroup per 16-row block, its waves split
 * K; M <= 16, K <= 8192); 2 = streaming with X shared through LDS, 1 row
 * block per wave; 3 = the same with 2 row blocks per wave; 4 = tiled, 256
 * rows x 64 columns per 8-wave workgroup (X staged in LDS); 5 = tiled, 256
 * rows x 128 columns; 6 = k-split (8-wave workgroups, one 512-k tile per
 * wave and K-split, each workgroup's row blocks all in flight; M <= 16, at
 * most K = 4096 per split and 8 row blocks per workgroup, i.e. N/16 <=
 * 8 * (CUs / splits)); 7 = streaming with X shared through LDS, 8 waves,
 * 1 row block x 32 columns per wave (each spliced k-step feeds both column
 * groups); 8 = the same with 2 row blocks per wave; 9 = k-ring (one 8-wave
 * workgroup per ceil(N/16 / CUs) row blocks, each wave a fixed K slice of X
 * in registers, a register ring over the row blocks; M <= 16, K <= 8192, at
 * most 8 row blocks per CU, no K-splits).  Variants 2-5, 7 and 8 handle any
 * M.  splits: 0 = automatic, else K-splits across workgroups (1..K/512;
 * variants 2-8).
 * Errors: as fp6_linear_plan, plus FP6_E_VALUE for a shape variant 1, 6 or
 * 9 does not cover.
 */
int fp6s_linear_plan(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                     int64_t N, int64_t K, int variant, int splits, void* stream);

/* fp6s_linear_plan_query -- host: the schedule fp6s_linear would use for
 * (M, N, K) on the current device (*variant 1..9, *splits).  One HIP query.
 * Errors: FP6_E_NULL, FP6_E_SHAPE (M >= 1, K % 512 == 0), FP6_E_HIP. */
int fp6s_linear_plan_query(int64_t M, int64_t N, int64_t K, int* variant, int* splits);

/* fp6s_dequant -- device, asynchronous: dense Wdq fp16 [N][K] (zeros at the
 * pruned positions) from the packed 2:4 buffer, with the same device splice
 * as fp6s_linear.  Errors: as fp6_dequant. */
int fp6s_dequant(const void* packed_W, const void* scales, void* W16, int64_t N, int64_t K,
                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP6S_AMD_H */
