/*
 * fp6.h -- C ABI of the MI355X (gfx950) weight-only FP6 linear layer (W6A16).
 *
 *   Y[M,N] = X[M,K] . dequant(W_fp6[N,K])^T
 *
 * X and Y are fp16, W is FP6 e3m2 (1 sign, 3 exponent, 2 mantissa bits,
 * bias 3, subnormals, no inf/NaN, max 28) with one fp16 scale per output row.
 * De-quantisation and the product run in one kernel, so no fp16 copy of W is
 * ever written to memory (TC-FPx explainer, duicuo.cn, section "redesigning
 * the kernel solution": one fused kernel instead of a de-quantise kernel plus
 * a matmul kernel; FP6 values are turned into FP16 and multiplied as FP16).
 * The weights are re-ordered and split into 2-bit and 4-bit pieces offline
 * (same section: bit-level pre-packing into aligned words, 6 = 2 + 4 bit
 * splitting, fragments re-ordered before run time).
 *
 * Conventions for every entry point:
 *   - All functions return an int status (enum fp6_status); FP6_OK == 0.
 *   - No function aborts, throws across the ABI or prints.
 *   - Argument checks happen on the host before any HIP call, so an invalid
 *     call never touches the GPU.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *     memory of the current HIP device (e.g. a torch CUDA tensor's data_ptr).
 *   - The caller owns every buffer it passes.  The library owns only the
 *     split-K workspace described at fp6_linear.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Device entry points only enqueue work on it and never
 *     synchronise it, except where stated.
 *
 * Size limits: 16 <= N <= 2^24 with N % 16 == 0; 256 <= K <= 2^24 with
 * K % 256 == 0; 0 <= M <= 2^24; N*K <= 2^36.  Violations give FP6_E_SHAPE.
 */
#ifndef FP6_AMD_H
#define FP6_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp6_status {
  FP6_OK = 0,
  FP6_E_NULL = 1,   /* a required pointer is NULL                           */
  FP6_E_SHAPE = 2,  /* M, N or K outside the limits above                   */
  FP6_E_ALIGN = 3,  /* a device pointer is not 16-byte aligned (scales: 2)  */
  FP6_E_CODE = 4,   /* a weight code is > 63                                */
  FP6_E_SCALE = 5,  /* a scale is not finite or |s| >= 16                   */
  FP6_E_SIZE = 6,   /* a caller buffer size does not match (fp6_linear_noalloc:
                       the plan needs more than the static scratch)         */
  FP6_E_HIP = 7,    /* a HIP runtime call or kernel launch failed           */
  FP6_E_VALUE = 8,  /* an input value is invalid (NaN/inf weight) or a plan
                       parameter is out of range                            */
};

/* Version of the packed weight layout produced by fp6_prepack (3).  The
 * kernels read this version only: a buffer packed by an earlier version is
 * packed again from its codes (fp6_prepack is deterministic). */
int fp6_pack_version(void);

/* Static, NUL-terminated text for a status code (never NULL). */
const char* fp6_status_string(int status);

/* Bytes of the packed buffer for an N x K weight: exactly N*K*3/4, or 0 if
 * (N, K) is outside the limits. */
size_t fp6_packed_bytes(int64_t N, int64_t K);

/*
 * fp6_quantize_rows -- host, synchronous, deterministic.
 * Quantises fp32 weights to e3m2 codes with one fp16 scale per row:
 *   s_n = fp16_RNE(max_k |W[n,k]| / 28)   (quotient in double, one rounding)
 *   c   = sign(W) << 5 | nearest e3m2 magnitude of |W / s_n| (double quotient;
 *         ties to the even code; >= 28 saturates to 28; rows with s_n == 0
 *         get all-zero codes).
 * W: host float32 [N][K] row-major, finite.  codes: host uint8 [N][K] out.
 * scales: host uint16 (fp16 bit patterns) [N] out.
 * Any N >= 1, K >= 1 (no tiling constraint).  Errors: FP6_E_NULL, FP6_E_SHAPE,
 * FP6_E_VALUE (non-finite W), FP6_E_SCALE (a row gives |s| >= 16); on error
 * the outputs are unspecified.  The pages do not describe quantisation; this
 * is the input preparation used by the tests and the benchmark.
 */
int fp6_quantize_rows(const float* W, int64_t N, int64_t K,
                      uint8_t* codes, uint16_t* scales);

/*
 * fp6_prepack -- host, synchronous, pure and deterministic (offline step).
 * Re-orders 6-bit codes into packed layout v3 (TC-FPx explainer, section
 * "redesigning the kernel solution": bit-level pre-packing and 2+4 splitting
 * before inference).
 *
 * codes:   host uint8 [N][K] row-major, every value in 0..63.
 * scales:  host uint16 fp16 bit patterns [N]; checked only (finite, |s| < 16,
 *          the range in which s * 2^12 is an exact fp16, which the fused
 *          kernel relies on); pass the same values to fp6_linear.
 * packed:  host out, packed_bytes == fp6_packed_bytes(N, K).
 * Errors: FP6_E_NULL, FP6_E_SHAPE, FP6_E_CODE, FP6_E_SCALE, FP6_E_SIZE.
 *
 * Packed layout v3 (fp6_pack_version() == 3).  Tiles of 16 rows x 256 k,
 * 3072 bytes each, k-block major: tile (nb, kb) starts at byte
 * (kb*(N/16) + nb)*3072, so the row blocks read at one k-block are adjacent.
 * Within a tile, local row r (0..15) and local k = 32*j + 8*g + i (k-step j
 * 0..7, lane group g 0..3, element i 0..7) belong to wave lane L = 16*g + r.
 * Each code c is split into a 2-bit piece (s, e2) = c >> 4 and a 4-bit piece
 * (e1 e0 m1 m0) = c & 15.  Element i is in group G = i/4 at byte E = i%4.
 *   bytes [0,1024):    2-bit plane.  Lane L's 16 bytes at 16*L are four
 *                      little-endian words; word j/2 covers k-steps j, j+1.
 *                      With rho = 4*(j%2) + 2*G, bit e2 is at
 *                      (4 + 8E + rho) mod 32 and bit s at (7 + 8E + rho) mod 32.
 *   bytes [1024,3072): 4-bit plane; k-steps 0..3 in the first 1024 bytes,
 *                      4..7 in the second.  Lane L's 16 bytes at 16*L hold
 *                      words j%4; element i is the nibble at bits
 *                      4*(2E + G) .. +3 (elements 0..3 in the low nibbles).
 * A wave reads one tile with three fully coalesced 16-byte-per-lane loads,
 * and each lane's words hold exactly the 8 k-values per k-step that a
 * 16x16x32 fp16 MFMA A-operand lane consumes.  The positions make the fp16
 * high bytes (s<<7)|(e2<<4)|nibble of four elements one and_or of the
 * 4-bit word with the rotated 2-bit word, spread onto fp16 pairs by one
 * byte permute per pair.  (Layout v1, the first version, placed the pieces
 * per fp16 pair instead; v2 changed only the bit positions; v3 only the
 * order of the tiles, which layouts v1 and v2 kept row-block major.)
 */
int fp6_prepack(const uint8_t* codes, const uint16_t* scales,
                int64_t N, int64_t K, void* packed, size_t packed_bytes);

/*
 * fp6_linear -- device, asynchronous on `stream` (the hot path).
 *   Y[m,n] = sum_k X[m,k] * Wdq[n,k],  Wdq[n,k] = fp16_RNE(v(c[n,k]) * s_n)
 * with fp32 accumulation and one final rounding to fp16 (IEEE RNE).  FP6-LLM
 * (arXiv 2401.14112) abstract: W6A16 linear layers on tensor cores; TC-FPx
 * explainer, section "redesigning the kernel solution": one fused kernel.
 *
 * X:        device fp16 [M][K] row-major, 16-byte aligned.
 * packed_W: device, the bytes of fp6_prepack(N, K) copied verbatim, 16-byte
 *           aligned.
 * scales:   device fp16 [N], the values given to fp6_prepack (unchecked here).
 * Y:        device fp16 [M][N] row-major, 16-byte aligned, must not overlap
 *           any input.
 * M == 0 is a no-op returning FP6_OK (X and Y may then be NULL).
 * Errors: FP6_E_NULL, FP6_E_SHAPE, FP6_E_ALIGN (before any HIP call);
 *         FP6_E_HIP if the launch or a workspace allocation fails.
 * Workspace: when the plan splits K (memory-bound small-M shapes) the library
 * keeps an fp32 partial-sum buffer and a self-resetting counter array per
 * (device, stream), allocated with hipMalloc on first need and grown on
 * demand.  A workspace that grows keeps its old buffers allocated until
 * fp6_release (launches in flight and graphs captured before the growth
 * still use them).  Results are bitwise deterministic: split partials are
 * summed in a fixed order.
 * A workspace is kept for every stream that ran a split plan, until
 * fp6_release (a process that creates many streams holds one per stream).
 * Concurrent calls on different streams are safe.  Calls on one stream from
 * several host threads are safe too: the library holds its lock from the
 * workspace lookup until the launch is enqueued, and the stream orders the
 * kernels.
 * HIP graph capture: nothing is allocated or cleared per call once the
 * stream's workspace exists, so make one call with the same shape and plan
 * on the capturing stream before capturing.  The captured launch keeps the
 * workspace's buffers; a later growth (a larger split-K plan on that
 * stream) leaves them allocated, so the graph stays valid until
 * fp6_release, which frees them (do not replay it after that).  Graphs
 * captured on a stream with the same buffers share them (partial sums and
 * arrival counters): replay such graphs one after another, never two at
 * once on different streams and never alongside eager split-K calls on the
 * capturing stream, or their partial sums mix.
 */
int fp6_linear(const void* X, const void* packed_W, const void* scales, void* Y,
               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp6_linear_noalloc -- fp6_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, plan, kernels and result bits as
 * fp6_linear, but split plans keep their fp32 partial sums and arrival
 * counters in a static device array of the library (64 MiB + 256 KiB, of
 * which the first 256 KiB are counters; each GPU holds its own copy until the process
 * ends) instead of a per-stream workspace: the call never calls hipMalloc,
 * hipFree or any allocating routine.  The first call on a device looks the
 * array up and clears its counters with a kernel on `stream`; split plans
 * leave them at zero.
 * Every call on a GPU shares that GPU's one array: calls that overlap on one
 * GPU (on different streams, or graphs replayed alongside eager calls) race
 * and give wrong sums.  Order them on one stream.
 * Errors: as fp6_linear, plus FP6_E_SIZE when the plan would need more
 * partial sums or counters than the array holds (no automatic plan does on a
 * 256-CU MI355X: at most 32 MiB for split-K plans, 64 MiB for stream-K).
 */
int fp6_linear_noalloc(const void* X, const void* packed_W, const void* scales, void* Y,
                       int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp6_linear_plan -- fp6_linear with the schedule forced (tuning and tests).
 * variant: 0 = automatic (what fp6_linear does), else one kernel
 *   configuration:
 *     1  streaming, 1 row block (16 rows) per wave, prefetch ring of 4 tiles
 *     2  streaming, 1 row block x 64 columns per wave, ring of 2 tiles
 *     3  streaming, 2 row blocks per wave, ring of 4 tiles
 *     4  streaming, 4 row blocks per wave, ring of 2 tiles
 *     5  tiled, 256 rows x 64 columns per 4-wave workgroup (X staged in LDS)
 *     6  tiled, 256 rows x 128 columns per 4-wave workgroup
 *     7  streaming, 1 row block per wave, ring of 8 tiles
 *     8  streaming, 2 row blocks per wave, ring of 6 tiles
 *     9  k-split persistent: one 8-wave workgroup per CU, waves split K and
 *        keep their X slice in registers; requires M <= 16 and at most
 *        8192 of K per K-split
 *    10  tiled, 256 rows x 128 columns per 8-wave workgroup (2 row blocks
 *        per wave, two waves per SIMD)
 *    11  tiled, 256 rows x 64 columns per 8-wave workgroup
 *    12  k-split persistent with 16 waves per workgroup (same limits as 9)
 *    13  k-slice: the waves of a workgroup (8 or 16, by K) split
 *        one row block's K, X streamed per half-tile; requires M <= 16,
 *        K <= 12288
 *    14  streaming, X tiles shared through LDS by the workgroup's 4 waves,
 *        2 row blocks per wave, ring of 4 tiles
 *    15  as 14 with 1 row block per wave
 *    16  as 14 with 8 waves per workgroup
 *    17  tiled, 256 rows x 64 columns per 8-wave workgroup, whole 256-k tiles
 *        per pipeline stage (one barrier per tile)
 *    18  as 15 with 8 waves per workgroup (each X tile shared by 8 waves)
 *    19  streaming with X in LDS, 8 waves, 2 row blocks x 32 columns per wave
 *        (each k-step of a row block spliced once for both column groups),
 *        ring of 2 tiles
 *    20  as 19 with 64 columns per wave
 *    21  as 19 with 1 row block per wave and a ring of 4 tiles
 *    22  as 20 with 1 row block per wave
 *    23  as 10 with the packed weights staged in LDS: every global load is
 *        a direct LDS load, the weights four half-tiles deep
 *    24  as 23 with 64 columns per workgroup
 *    25  as 10, stream-K: one workgroup per CU, each running an equal
 *        contiguous range of (tile, 128-k half-tile) units; a tile's pieces
 *        meet in the fixed-order fix-up
 *    26  k-ring: one 8-wave workgroup per P consecutive row blocks and
 *        K-split; each wave keeps a fixed 1/8 of its split's K of X in
 *        registers and streams its tiles of every row block through a
 *        register ring; one fixed-order cross-wave sum, then the split-K
 *        fix-up.  Requires M <= 16, at most 8192 of K per split (splits 0 =
 *        the fewest that fit) and P = ceil(N/16 * splits / CUs) <= 8
 *   Streaming and tiled kernels handle any M (16-column groups per pass).
 * splits:  0 = automatic, else the number of K-splits across workgroups
 *          (1..K/256; must be 0 or 1 for variant 13, 0 for variant 25).
 * The result equals fp6_linear's up to fp32 summation order.
 * Errors: as fp6_linear, plus FP6_E_VALUE for an unknown variant, a split
 * count out of range, or a shape that variant 9, 12, 13 or 26 does not
 * cover.
 */
int fp6_linear_plan(const void* X, const void* packed_W, const void* scales, void* Y,
                    int64_t M, int64_t N, int64_t K, int variant, int splits,
                    void* stream);

/*
 * fp6_linear_plan_query -- host; reports the schedule fp6_linear would use
 * for (M, N, K) on the current device: *variant (1..26, see fp6_linear_plan)
 * and *splits (K-splits across workgroups, 1 = none; for variant 25 the
 * number of stream-K workgroups).  Makes one HIP query
 * (device id and CU count).  Errors: FP6_E_NULL, FP6_E_SHAPE (M must be
 * >= 1 here), FP6_E_HIP.
 */
int fp6_linear_plan_query(int64_t M, int64_t N, int64_t K, int* variant, int* splits);

/*
 * fp6_dequant -- device, asynchronous; test and inspection export.
 * Writes Wdq fp16 [N][K] row-major using the same splice-and-scale device
 * function as fp6_linear (TC-FPx explainer, section "redesigning the kernel
 * solution": FP6 weights rebuilt as FP16 in registers).  W16 must be 16-byte
 * aligned and hold N*K halves.  Errors: FP6_E_NULL, FP6_E_SHAPE,
 * FP6_E_ALIGN, FP6_E_HIP.
 */
int fp6_dequant(const void* packed_W, const void* scales, void* W16,
                int64_t N, int64_t K, void* stream);

/* Frees every split-K workspace the library holds, synchronising each device
 * that holds one first (work still in flight may use it).  Returns FP6_OK, or
 * FP6_E_HIP if a device could not be synchronised or a buffer freed (the
 * buffers not freed are kept and a later call retries them). */
int fp6_release(void);

#ifdef __cplusplus
}
#endif
#endif /* FP6_AMD_H */
