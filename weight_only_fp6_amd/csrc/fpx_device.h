// Kernels of the fused FPx weight-only linear layer for gfx950 (MI355X),
// templated on the weight format, plus their host-side launchers.  Included
// by one translation unit per format (fpx_kern_<format>.hip).
//
// FP6-LLM (arXiv 2401.14112), abstract: the two costs of FP6 weights on GPUs
// are irregular-width memory access and de-quantisation overhead, and one
// kernel scheme should serve float weights of several widths.  TC-FPx
// explainer (duicuo.cn), section "redesigning the kernel solution": one
// kernel de-quantises in registers and feeds FP16 matrix units; weights are
// pre-split into power-of-two pieces so the splice is a few bit operations.
//
// gfx950 design:
//  * A wave owns 16 weight rows (one 16x16x32 MFMA A-operand row block) and a
//    range of 256-wide k-tiles.  Per tile it issues two or three coalesced
//    loads per lane (1 KiB per wave instruction for a 16-byte load), exactly
//    the bits of its 64 codes.
//  * Splice (FP6 e3m2): for the fp16 pair (2r, 2r+1) of k-step j,
//      bits = ((d4 shifted into bits 8..11 / 24..27) & 0x0F000F00)
//           | (rotr(d2, 2p) & 0x90009000),      p = 4*(j%2) + r
//    which is the fp16 pattern of v(c) * 2^-12 (sign at bit 15, e2 at bit 12,
//    e1 e0 m1 m0 at bits 11..8; e3m2 subnormals become fp16 subnormals).  The
//    other formats use the same scheme with their own masks and rotations.
//  * Scale fold: one v_pk_mul_f16 by s_n * 2^12 (e3m2), an exact fp16 for
//    |s| < 16, so the single rounding gives fp16_RNE(v * s_n) bit for bit.
//  * fp32 MFMA accumulation (v_mfma_f32_16x16x32_f16), A = weights (rows n),
//    B = X^T (columns m), so the accumulator tile is Y^T.
//  * Split-K for the memory-bound small-M regime: each split writes an fp32
//    partial tile; the last split to arrive (agent-scope counter) sums the
//    partials in split order and stores fp16 Y, then resets the counter.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fp6.h"
#include "fp6_limits.h"
#include "fpx_launch.h"

namespace {

using fpx::kKsMaxTiles;
using fpx::kKsliceMaxTiles;

inline int64_t fpx_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveSize = 64;

// ---------------------------------------------------------------------------
// Weight formats.  Every format packs a 16-row x 256-k tile so that wave lane
// L = 16g + r holds the codes of row r at k = 32j + 8g + i (k-step j, element
// i): the A-operand order of v_mfma_f32_16x16x32_f16.  A lane rebuilds each
// pair of fp16 weights with a few bit operations (FP4: the gfx950 FP4
// conversion instruction) and one v_pk_mul_f16 by its row's scale.
//   FP6 e3m2: fp16 pattern (s<<15)|(c&31)<<8 = v * 2^-12; scale factor s*2^12
//   FP6 e2m3: (s<<15)|(c&31)<<7 = v * 2^-14;            scale factor s*2^14
//   FP5 e2m2: (s<<15)|(c&15)<<8 = v * 2^-14;            scale factor s*2^14
//   FP4 e2m1: converted exactly to v;                    scale factor s
// Each scale factor is an exact fp16 for the scales fp6_prepack/fpx_prepack
// accept, so the one rounding of the multiply gives fp16_RNE(v * s).
// Tiles follow one another k-tile by k-tile: tile (row block nb, k-tile kt)
// is tile number kt * (N / 16) + nb, so the row blocks that a wave or a
// workgroup reads at one k-tile lie side by side in memory.
// ---------------------------------------------------------------------------
enum : int { kE3M2 = 0, kE2M3 = 1, kE2M2 = 2, kE2M1 = 3 };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Packed registers of one tile (8 k-steps) and one half-tile (4 k-steps) of
// one row block, per lane.
struct TileFp6 { u32x4 q2, q4a, q4b; };   // 2-bit words (2 k-steps each), 4-bit words
struct HalfFp6 { u32x2 q2; u32x4 q4; };
struct TileFp5 { u32x4 q4a, q4b; u32x2 q1; };  // 4-bit words, 1-bit words (4 k-steps each)
struct HalfFp5 { uint32_t q1; u32x4 q4; };
struct TileFp4 { u32x4 q4a, q4b; };
struct HalfFp4 { u32x4 q4; };

// 6-bit formats, one k-step: 8 fp16 weights (elements 8g..8g+7 of row r)
// from the 2-bit word d2 (k-steps 2*(j/2), +1) and the 4-bit word d4.
//   e3m2: the fp16 pattern of v * 2^-12 has all its bits in the high byte:
//         (s<<7) | (e2<<4) | (e1 e0 m1 m0).  The 4-bit word holds elements
//         0..3 in the low nibbles and 4..7 in the high nibbles of its bytes;
//         for group G (elements 4G..4G+3) the 2-bit word rotated right by
//         4*(j%2) + 2G has e2 and s of element 4G+E at bits 4 and 7 of byte
//         E.  So one and_or builds the four high bytes of a group, and one
//         v_perm_b32 per pair spreads two of them onto the fp16 halves.
//   e2m3: pair p has e1,s at bits b, b+4 (+16), b = [0,1,2,3,8,9,10,11][p];
//         rotr(d2, (b-11) mod 32) lands them on fp16 bits 11 and 15; the
//         4-bit word holds element i in nibble slot i/2 + 4*(i%2), so one
//         shift per pair q moves elements 2q and 2q+1 onto both fp16 halves.
template <int F, int JODD>
__device__ __forceinline__ half8v splice6(uint32_t d2, uint32_t d4, half2v s2) {
  uint32_t t0, t1, t2, t3;
  if constexpr (F == kE3M2) {
    constexpr uint32_t kNib = 0x0F0F0F0Fu, kSE = 0x90909090u;
    // v_perm_b32 selectors: bytes (1, zero, 0, zero) and (3, zero, 2, zero).
    constexpr uint32_t kLo = 0x010C000Cu, kHi = 0x030C020Cu;
    const uint32_t wa = (d4 & kNib) | (__builtin_amdgcn_alignbit(d2, d2, 4 * JODD) & kSE);
    const uint32_t wb = ((d4 >> 4) & kNib) | (__builtin_amdgcn_alignbit(d2, d2, 4 * JODD + 2) & kSE);
    t0 = __builtin_amdgcn_perm(wa, wa, kLo);
    t1 = __builtin_amdgcn_perm(wa, wa, kHi);
    t2 = __builtin_amdgcn_perm(wb, wb, kLo);
    t3 = __builtin_amdgcn_perm(wb, wb, kHi);
  } else {
    static_assert(F == kE2M3, "6-bit formats: e3m2, e2m3");
    constexpr uint32_t kM4 = 0x07800780u, kM2 = 0x88008800u;
    constexpr int r0 = JODD ? 29 : 21;  // (b - 11) mod 32 for pair 0 of this k-step
    t0 = ((d4 << 7) & kM4) | (__builtin_amdgcn_alignbit(d2, d2, r0) & kM2);
    t1 = ((d4 << 3) & kM4) | (__builtin_amdgcn_alignbit(d2, d2, r0 + 1) & kM2);
    t2 = ((d4 >> 1) & kM4) | (__builtin_amdgcn_alignbit(d2, d2, r0 + 2) & kM2);
    t3 = ((d4 >> 5) & kM4) | (__builtin_amdgcn_alignbit(d2, d2, (r0 + 3) & 31) & kM2);
  }
  const half2v h0 = __builtin_bit_cast(half2v, t0) * s2;
  const half2v h1 = __builtin_bit_cast(half2v, t1) * s2;
  const half2v h2 = __builtin_bit_cast(half2v, t2) * s2;
  const half2v h3 = __builtin_bit_cast(half2v, t3) * s2;
  half8v a;
  a[0] = h0[0]; a[1] = h0[1]; a[2] = h1[0]; a[3] = h1[1];
  a[4] = h2[0]; a[5] = h2[1]; a[6] = h3[0]; a[7] = h3[1];
  return a;
}

// FP5 e2m2, k-step j: the fp16 pattern of v * 2^-14 has all its bits in the
// high byte too, (s<<7) | (e1 e0 m1 m0).  The 4-bit word is ordered as
// e3m2's; the 1-bit word d1 (k-steps 4*(j/4)..+3) rotated right by
// 2*(j%4) + G has the sign of element 4G+E at bit 7 of byte E.  So the
// e3m2 form applies: one and_or per group, one v_perm_b32 per pair.
template <int JM4>
__device__ __forceinline__ half8v splice5(uint32_t d1, uint32_t d4, half2v s2) {
  constexpr uint32_t kNib = 0x0F0F0F0Fu, kS = 0x80808080u;
  constexpr uint32_t kLo = 0x010C000Cu, kHi = 0x030C020Cu;  // as in splice6
  const uint32_t wa = (d4 & kNib) | (__builtin_amdgcn_alignbit(d1, d1, 2 * JM4) & kS);
  const uint32_t wb = ((d4 >> 4) & kNib) | (__builtin_amdgcn_alignbit(d1, d1, 2 * JM4 + 1) & kS);
  const uint32_t t0 = __builtin_amdgcn_perm(wa, wa, kLo);
  const uint32_t t1 = __builtin_amdgcn_perm(wa, wa, kHi);
  const uint32_t t2 = __builtin_amdgcn_perm(wb, wb, kLo);
  const uint32_t t3 = __builtin_amdgcn_perm(wb, wb, kHi);
  const half2v h0 = __builtin_bit_cast(half2v, t0) * s2;
  const half2v h1 = __builtin_bit_cast(half2v, t1) * s2;
  const half2v h2 = __builtin_bit_cast(half2v, t2) * s2;
  const half2v h3 = __builtin_bit_cast(half2v, t3) * s2;
  half8v a;
  a[0] = h0[0]; a[1] = h0[1]; a[2] = h1[0]; a[3] = h1[1];
  a[4] = h2[0]; a[5] = h2[1]; a[6] = h3[0]; a[7] = h3[1];
  return a;
}

// FP4 e2m1, one k-step: byte q of the 4-bit word holds elements 2q (low
// nibble) and 2q+1; v_cvt_scalef32_pk_f16_fp4 with scale 1 converts them
// exactly (it applies only the exponent of its scale operand).
__device__ __forceinline__ half8v splice4(uint32_t d4, half2v s2) {
  const half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4, 1.0f, 0) * s2;
  const half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4, 1.0f, 1) * s2;
  const half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4, 1.0f, 2) * s2;
  const half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d4, 1.0f, 3) * s2;
  half8v a;
  a[0] = h0[0]; a[1] = h0[1]; a[2] = h1[0]; a[3] = h1[1];
  a[4] = h2[0]; a[5] = h2[1]; a[6] = h3[0]; a[7] = h3[1];
  return a;
}

// Direct global -> LDS load of BYTES (4 or 16) per lane: lane i's bytes land
// at lds + BYTES*i (lds is wave-uniform).
template <int BYTES>
__device__ __forceinline__ void lds_load(const void* src, void* lds) {
  static_assert(BYTES == 4 || BYTES == 16, "direct LDS loads of 4 or 16 bytes per lane");
  auto* dst = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds));
  if constexpr (BYTES == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
}

// Weight loads.  With NT the load carries the non-temporal hint: the
// memory-bound kernels read each packed byte once per launch, and streaming
// them past the caches (instead of displacing X and the next launch's
// lines) measured 2-8% faster there (Llama-70B MLP M=16 32.0 -> 31.1 us,
// Llama-7B attention 4.73 -> 4.37 us).  Kernels whose column passes read
// the same weights again keep plain loads (OPT-30B QKV M=256, two 128-
// column tiles: 6% slower with the hint).
template <bool NT, typename T>
__device__ __forceinline__ T ldw(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Format traits.  kTileQuads: 16-byte units per packed tile; kHalfLoads,
// kTileLoads: load instructions per half-tile and per tile (the tiled
// kernels' wait counts depend on them).  load/load_half take the lane's pointer into the tile (tile + lane,
// in 16-byte units) and the lane index.
template <int F> struct Fmt;

template <int F>
struct Fp6Fmt {
  static constexpr int kTileQuads = 192;
  static constexpr int kHalfLoads = 2;
  static constexpr int kTileLoads = 3;
  static constexpr float kScaleFactor = F == kE3M2 ? 4096.0f : 16384.0f;
  using Tile = TileFp6;
  using Half = HalfFp6;
  template <bool NT = false>
  __device__ static void load(Tile& t, const u32x4* p, int) {
    t.q2 = ldw<NT>(p);
    t.q4a = ldw<NT>(p + 64);
    t.q4b = ldw<NT>(p + 128);
  }
  __device__ static void load_half(Half& h, const u32x4* p, int hh, int) {
    h.q2 = reinterpret_cast<const u32x2*>(p)[hh];
    h.q4 = p[64 + 64 * hh];
  }
  template <int J>
  __device__ static half8v step(const Tile& t, half2v s2) {
    return splice6<F, J & 1>(t.q2[J >> 1], J < 4 ? t.q4a[J & 3] : t.q4b[J & 3], s2);
  }
  template <int JJ>
  __device__ static half8v half_step(const Half& h, half2v s2) {
    return splice6<F, JJ & 1>(h.q2[JJ >> 1], h.q4[JJ], s2);
  }
  // LDS staging of half hh of one row block's tile (lane pointer p), by
  // direct LDS loads: the lane's 4-bit words (16 B) at 16*lane, its two
  // 2-bit words at 1024 + 4*lane and 1280 + 4*lane of the wave-uniform
  // region `lds` (kStageBytes).
  static constexpr int kStageBytes = 1536;
  static constexpr int kStageLoads = 3;
  __device__ static void stage_half(char* lds, const u32x4* p, int hh, int) {
    lds_load<16>(p + 64 + 64 * hh, lds);
    lds_load<4>(reinterpret_cast<const uint32_t*>(p) + 2 * hh, lds + 1024);
    lds_load<4>(reinterpret_cast<const uint32_t*>(p) + 2 * hh + 1, lds + 1280);
  }
  __device__ static void read_half(Half& h, const char* lds, int lane) {
    h.q4 = reinterpret_cast<const u32x4*>(lds)[lane];
    h.q2[0] = reinterpret_cast<const uint32_t*>(lds + 1024)[lane];
    h.q2[1] = reinterpret_cast<const uint32_t*>(lds + 1280)[lane];
  }
};
template <> struct Fmt<kE3M2> : Fp6Fmt<kE3M2> {};
template <> struct Fmt<kE2M3> : Fp6Fmt<kE2M3> {};

template <>
struct Fmt<kE2M2> {
  static constexpr int kTileQuads = 160;
  static constexpr int kHalfLoads = 2;
  static constexpr int kTileLoads = 3;
  static constexpr float kScaleFactor = 16384.0f;
  using Tile = TileFp5;
  using Half = HalfFp5;
  // 4-bit plane in 16-byte units 0..127 of the tile, 1-bit plane as 8 bytes
  // per lane from byte 2048.
  __device__ static const u32x2* plane1(const u32x4* p, int lane) {
    return reinterpret_cast<const u32x2*>(p) - lane + 256;
  }
  template <bool NT = false>
  __device__ static void load(Tile& t, const u32x4* p, int lane) {
    t.q4a = ldw<NT>(p);
    t.q4b = ldw<NT>(p + 64);
    t.q1 = ldw<NT>(plane1(p, lane));
  }
  __device__ static void load_half(Half& h, const u32x4* p, int hh, int lane) {
    h.q1 = reinterpret_cast<const uint32_t*>(plane1(p, lane))[hh];
    h.q4 = p[64 * hh];
  }
  template <int J>
  __device__ static half8v step(const Tile& t, half2v s2) {
    return splice5<J & 3>(t.q1[J >> 2], J < 4 ? t.q4a[J & 3] : t.q4b[J & 3], s2);
  }
  template <int JJ>
  __device__ static half8v half_step(const Half& h, half2v s2) {
    return splice5<JJ>(h.q1, h.q4[JJ], s2);
  }
  // LDS staging (see Fp6Fmt): 4-bit words at 16*lane, 1-bit word at 1024 + 4*lane.
  static constexpr int kStageBytes = 1280;
  static constexpr int kStageLoads = 2;
  __device__ static void stage_half(char* lds, const u32x4* p, int hh, int lane) {
    lds_load<16>(p + 64 * hh, lds);
    lds_load<4>(reinterpret_cast<const uint32_t*>(plane1(p, lane)) + hh, lds + 1024);
  }
  __device__ static void read_half(Half& h, const char* lds, int lane) {
    h.q4 = reinterpret_cast<const u32x4*>(lds)[lane];
    h.q1 = reinterpret_cast<const uint32_t*>(lds + 1024)[lane];
  }
};

template <>
struct Fmt<kE2M1> {
  static constexpr int kTileQuads = 128;
  static constexpr int kHalfLoads = 1;
  static constexpr int kTileLoads = 2;
  static constexpr float kScaleFactor = 1.0f;
  using Tile = TileFp4;
  using Half = HalfFp4;
  template <bool NT = false>
  __device__ static void load(Tile& t, const u32x4* p, int) {
    t.q4a = ldw<NT>(p);
    t.q4b = ldw<NT>(p + 64);
  }
  __device__ static void load_half(Half& h, const u32x4* p, int hh, int) { h.q4 = p[64 * hh]; }
  template <int J>
  __device__ static half8v step(const Tile& t, half2v s2) {
    return splice4(J < 4 ? t.q4a[J & 3] : t.q4b[J & 3], s2);
  }
  template <int JJ>
  __device__ static half8v half_step(const Half& h, half2v s2) {
    return splice4(h.q4[JJ], s2);
  }
  // LDS staging (see Fp6Fmt): 4-bit words at 16*lane.
  static constexpr int kStageBytes = 1024;
  static constexpr int kStageLoads = 1;
  __device__ static void stage_half(char* lds, const u32x4* p, int hh, int) { lds_load<16>(p + 64 * hh, lds); }
  __device__ static void read_half(Half& h, const char* lds, int lane) {
    h.q4 = reinterpret_cast<const u32x4*>(lds)[lane];
  }
};

template <int F>
__device__ __forceinline__ half2v scale2_of(_Float16 s) {
  if constexpr (Fmt<F>::kScaleFactor != 1.0f) s = s * static_cast<_Float16>(Fmt<F>::kScaleFactor);
  half2v s2;
  s2[0] = s;
  s2[1] = s;
  return s2;
}
template <int F>
__device__ __forceinline__ half2v row_scale2(const _Float16* scales, int64_t n) {
  return scale2_of<F>(scales[n]);
}

// ---------------------------------------------------------------------------
// De-quantisation export: one wave per tile, Wdq fp16 [N][K] row-major.
// ---------------------------------------------------------------------------
template <int F>
__global__ __launch_bounds__(256) void fp6_dequant_kernel(const u32x4* __restrict__ wp,
                                                          const _Float16* __restrict__ scales,
                                                          _Float16* __restrict__ w16,
                                                          int64_t N, int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t ktiles = K >> 8;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (tile >= (N >> 4) * ktiles) return;
  const int64_t nblocks = N >> 4;
  const int64_t kt = tile / nblocks, nb = tile - kt * nblocks;  // k-tile-major order
  const int r = lane & 15, g = lane >> 4;
  typename Fmt<F>::Tile t;
  Fmt<F>::load(t, wp + tile * Fmt<F>::kTileQuads + lane, lane);
  const int64_t n = nb * 16 + r;
  const half2v s2 = row_scale2<F>(scales, n);
  half8v* out = reinterpret_cast<half8v*>(w16 + n * K + kt * 256 + 8 * g);
  out[0] = Fmt<F>::template step<0>(t, s2);
  out[4] = Fmt<F>::template step<1>(t, s2);
  out[8] = Fmt<F>::template step<2>(t, s2);
  out[12] = Fmt<F>::template step<3>(t, s2);
  out[16] = Fmt<F>::template step<4>(t, s2);
  out[20] = Fmt<F>::template step<5>(t, s2);
  out[24] = Fmt<F>::template step<6>(t, s2);
  out[28] = Fmt<F>::template step<7>(t, s2);
}

// ---------------------------------------------------------------------------
// Split-K fix-up.  Every split of a work unit stores its fp32 accumulators
// with device-scope (sc1) 16-byte stores, waits for them to complete, then
// bumps the unit's counter with a device-scope atomic.  The split that sees
// count splits-1 is the last one: it reads the other partials with
// device-scope 16-byte loads, sums all splits in split order
// (deterministic), and resets the counter for the next call.  Device-scope
// accesses keep the partials coherent across the XCDs' L2 caches without
// any whole-cache write-back or invalidate (which agent-scope fences would
// issue in every wave).  The accesses go through a buffer resource over the
// unit's partials (sc1 is a cache-policy bit of buffer instructions), one
// dwordx4 per lane per accumulator: a quarter of the instructions of
// per-component stores.  Partial layout: [unit][split][acc i][lane] float4,
// so each instruction moves 1 KB contiguous; split s starts piece_quads
// 16-byte units after split s-1 (NACC*64 when a unit's splits are adjacent;
// larger when other units' slots sit between them).
// With kProbeFirst (for kernels whose last split has the most work and so
// usually finishes last), a split first reads the counter: if every other
// split has already stored (they count only after their stores complete),
// it is the last one and goes straight to the sum without storing its own
// partial or counting.  Otherwise it stores and counts as above.  Exactly
// one split finishes either way: one that sees splits-1 is the only split
// that has not counted, and a split whose count returns splits-1 was
// preceded by the counts of all others.
// ---------------------------------------------------------------------------
template <int NACC, bool kProbeFirst = false>
__device__ __forceinline__ bool splitk_fixup(float4v (&acc)[NACC], float* __restrict__ unit_part,
                                             unsigned* __restrict__ counter, int split, int splits,
                                             int lane, int piece_quads = NACC * 64) {
  constexpr int kSc1 = 16;                 // cache policy: device scope
  constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer, gfx9 family
  // The buffer spans exactly this unit's splits: the last one ends NACC*1 KB
  // after its start.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      unit_part, static_cast<short>(0), ((splits - 1) * piece_quads + NACC * 64) * 16, kRsrcWord3);
  bool last = false;
  if constexpr (kProbeFirst) {
    const unsigned seen = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    last = seen == static_cast<unsigned>(splits - 1);
  }
  if (!last) {
#pragma unroll
    for (int i = 0; i < NACC; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i]), rsrc,
                                             (split * piece_quads + i * 64 + lane) * 16, 0, kSc1);
    __builtin_amdgcn_s_waitcnt(0);  // the partial stores have completed
    unsigned prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != static_cast<unsigned>(splits - 1)) return false;
  }
  float4v sum[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) sum[i] = float4v{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    if (s == split) {
#pragma unroll
      for (int i = 0; i < NACC; ++i) sum[i] += acc[i];
    } else {
      u32x4 v[NACC];
#pragma unroll
      for (int i = 0; i < NACC; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (s * piece_quads + i * 64 + lane) * 16, 0, kSc1);
#pragma unroll
      for (int i = 0; i < NACC; ++i) sum[i] += __builtin_bit_cast(float4v, v[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = sum[i];
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Workgroup-index arithmetic in 32 bits: every operand (workgroup index,
// split count, tile and group counts, split * k-tiles) stays below 2^31, and
// a 64-bit division by a runtime value is a long software sequence that
// delays a kernel's first loads.  Division by 1 (no K-split) is skipped.
__device__ __forceinline__ uint32_t udiv32(uint32_t a, uint32_t b) { return b == 1 ? a : a / b; }
__device__ __forceinline__ uint32_t umod32(uint32_t a, uint32_t b) { return b == 1 ? 0 : a - (a / b) * b; }

// Store one 16x16 accumulator block (Y^T layout: lane holds Y[m][n0+4g .. +3]).
__device__ __forceinline__ void store_y_block(_Float16* __restrict__ Y, const float4v& v, int64_t m,
                                              int64_t M, int64_t N, int64_t n0, int g) {
  if (m >= M) return;
  half4v o;
  o[0] = static_cast<_Float16>(v[0]);
  o[1] = static_cast<_Float16>(v[1]);
  o[2] = static_cast<_Float16>(v[2]);
  o[3] = static_cast<_Float16>(v[3]);
  *reinterpret_cast<half4v*>(Y + m * N + n0 + 4 * g) = o;
}

// Sum of the W partial 16x16 tiles in LDS, in wave order (deterministic).
// The reads are issued 8 at a time before their adds, so their latencies
// overlap without holding all W tiles in registers.
template <int W>
__device__ __forceinline__ float4v reduce_waves(const float4v (&red)[W][64], int lane) {
  constexpr int kChunk = W < 8 ? W : 8;
  static_assert(W % kChunk == 0, "wave count must be a multiple of the chunk");
  float4v sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w0 = 0; w0 < W; w0 += kChunk) {
    float4v v[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) v[i] = red[w0 + i][lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) sum = (w0 + i == 0) ? v[i] : sum + v[i];
  }
  return sum;
}

// ---------------------------------------------------------------------------
// Streaming fused kernel (memory-bound regime).
// Work unit = (m-group of 16*MB columns, row group of A row blocks, K-split).
// A workgroup holds 4 waves = 4 consecutive row groups with the same m-group
// and split, so they read the same X slice (L1/L2 reuse).  Each wave keeps a
// ring of D packed tiles per row block in flight (3 x 16 B per lane per tile)
// and the X fragments of the next tile, splices each k-step once and reuses
// it for MB MFMAs; each X fragment is reused for A row blocks.
// ---------------------------------------------------------------------------
template <int F, int A>
struct WStage {
  typename Fmt<F>::Tile t[A];
};

template <int MB>
struct XStage {
  half8v b[8][MB];
};

template <int F, int A, int MB, int D>
__global__ __launch_bounds__(256) void fp6_gemm_stream(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  static_assert(D % 2 == 0, "X double buffer indexes by parity");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int64_t ngroups = (nblocks + A - 1) / A;
  const int64_t gquads = (ngroups + 3) >> 2;
  const uint32_t b = udiv32(blockIdx.x, splits);
  const int split = static_cast<int>(umod32(blockIdx.x, splits));
  const uint32_t bq = udiv32(b, static_cast<uint32_t>(gquads));
  const int64_t gq = b - bq * static_cast<uint32_t>(gquads);
  const int64_t mg = bq + mg_base;
  const int64_t rg = gq * 4 + wave;
  if (rg >= ngroups) return;
  const int64_t kt0 = udiv32(split * static_cast<uint32_t>(ktiles), splits);
  const int64_t kt1 = udiv32((split + 1) * static_cast<uint32_t>(ktiles), splits);
  const int r = lane & 15, g = lane >> 4;

  // Row blocks of this wave; a ragged last group repeats the last block and
  // drops its result.
  const u32x4* w[A];
  half2v s2[A];
#pragma unroll
  for (int a = 0; a < A; ++a) {
    int64_t nb = rg * A + a;
    if (nb >= nblocks) nb = nblocks - 1;
    w[a] = wp + nb * Fmt<F>::kTileQuads + lane;
    s2[a] = row_scale2<F>(scales, nb * 16 + r);
  }
  // B operand rows m = (mg*MB + mb)*16 + r; rows >= M read row M-1 (their
  // accumulator columns are never stored).
  const _Float16* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int64_t m = (mg * MB + mb) * 16 + r;
    if (m >= M) m = M - 1;
    xrow[mb] = X + m * K + 8 * g;
  }

  float4v acc[A * MB];
#pragma unroll
  for (int i = 0; i < A * MB; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](WStage<F, A>& st, int64_t kt) {
#pragma unroll
    for (int a = 0; a < A; ++a) {
      Fmt<F>::template load<MB == 1>(st.t[a], w[a] + kt * kstr, lane);
    }
  };
  auto load_x = [&](XStage<MB>& xs, int64_t kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        xs.b[j][mb] = *reinterpret_cast<const half8v*>(xrow[mb] + kt * 256 + 32 * j);
  };
  auto mac = [&](const WStage<F, A>& st, const XStage<MB>& xs) {
#define FP6_STEP(J)                                                                   \
  _Pragma("unroll") for (int a = 0; a < A; ++a) {                                     \
    const half8v av = Fmt<F>::template step<J>(st.t[a], s2[a]);     \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) acc[a * MB + mb] =              \
        __builtin_amdgcn_mfma_f32_16x16x32_f16(av, xs.b[J][mb], acc[a * MB + mb], 0, 0, 0); \
  }
    FP6_STEP(0) FP6_STEP(1) FP6_STEP(2) FP6_STEP(3)
    FP6_STEP(4) FP6_STEP(5) FP6_STEP(6) FP6_STEP(7)
#undef FP6_STEP
  };

  // Steady state: a branch-free loop over groups of D tiles, every load
  // issued unconditionally (tile index clamped to the unit's last tile; the
  // few extra loads at the end hit in cache).  The loads in flight are then
  // the same on every path, so the in-order vmcnt waits only ever wait for
  // the stage being consumed.  The last (< D) tiles run in an explicit tail.
  WStage<F, A> ring[D];
  XStage<MB> xs[2];
  const int64_t klast = kt1 > kt0 ? kt1 - 1 : kt0;
  auto clampk = [&](int64_t t) { return t < klast ? t : klast; };
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(ring[d], clampk(kt0 + d));
  load_x(xs[0], clampk(kt0));
  int64_t kt = kt0;
  for (; kt + D <= kt1; kt += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t t = kt + d;
      load_x(xs[(d + 1) & 1], clampk(t + 1));
      mac(ring[d], xs[d & 1]);
      load_w(ring[d], clampk(t + D));
    }
  }
  // Tail: tiles kt .. kt1-1 sit in ring[0 .. kt1-kt-1]; xs[0] holds X(kt).
  const int64_t rem = kt1 - kt;
#pragma unroll
  for (int d = 0; d + 1 < D; ++d) {
    if (d < rem) {
      load_x(xs[(d + 1) & 1], clampk(kt + d + 1));
      mac(ring[d], xs[d & 1]);
    }
  }

  if (splits > 1) {
    const int64_t unit = mg * ngroups + rg;
    float* unit_part = part + unit * static_cast<int64_t>(splits) * (A * MB * 256);
    if (!splitk_fixup<A * MB>(acc, unit_part, counters + unit, split, splits, lane)) return;
  }
#pragma unroll
  for (int a = 0; a < A; ++a) {
    const int64_t nb = rg * A + a;
    if (nb >= nblocks) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      store_y_block(Y, acc[a * MB + mb], (mg * MB + mb) * 16 + r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// Streaming kernel with X shared through LDS (memory-bound regime, M <= 16
// per m-group).  As fp6_gemm_stream, a wave streams A row blocks over a K
// range through a register ring of D packed tiles, but the NW waves of a
// workgroup (same K range, different row groups) share X: each X tile
// (16 rows x 256 k) is loaded once per workgroup into a 2-slot LDS ring
// (rows XOR-swizzled in 16-byte units, so the B-fragment reads are free of
// bank conflicts), one barrier per tile.  This cuts X's L2->CU traffic by NW.
//
// Vector-memory loads complete in issue order (one vmcnt counter), so a load
// that is needed soon must not be issued after loads that are needed late:
// waiting for it would also wait for them.  X therefore travels at the same
// prefetch distance D as the weights, through a register ring of D stages
// (X(t+D) is issued just before W(t+D), at the top of iteration t, and is
// written to LDS in iteration t+D-1).  Every wait then covers D-1 tiles of
// work instead of one.
//
// MB > 1: a workgroup covers MB groups of 16 columns (X tile MB*16 rows);
// each k-step of a row block is spliced once and feeds MB MFMAs, so the
// weights are streamed once for up to 16*MB columns.
// ---------------------------------------------------------------------------
template <int F, int A, int D, int NW, int MB = 1>
__global__ __launch_bounds__(64 * NW) void fp6_gemm_xlds(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  static_assert(D % 2 == 0, "the LDS slot of a tile is its parity");
  constexpr int kThreads = 64 * NW;
  constexpr int kChunks = MB * 16 * 32;                 // 16-byte units per X tile
  constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) half8v xs[2][kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int64_t ngroups = (nblocks + A - 1) / A;
  const int64_t gsets = (ngroups + NW - 1) / NW;
  const uint32_t b = udiv32(blockIdx.x, splits);
  const int split = static_cast<int>(umod32(blockIdx.x, splits));
  const uint32_t bq = udiv32(b, static_cast<uint32_t>(gsets));
  const int64_t gs = b - bq * static_cast<uint32_t>(gsets);
  const int64_t mg = bq + mg_base;
  const int64_t rg_raw = gs * NW + wave;
  const bool wave_active = rg_raw < ngroups;
  const int64_t rg = wave_active ? rg_raw : ngroups - 1;  // idle waves still join barriers
  const int64_t kt0 = udiv32(split * static_cast<uint32_t>(ktiles), splits);
  const int64_t kt1 = udiv32((split + 1) * static_cast<uint32_t>(ktiles), splits);
  const int r = lane & 15, g = lane >> 4;

  const u32x4* w[A];
  half2v s2[A];
#pragma unroll
  for (int a = 0; a < A; ++a) {
    int64_t nb = rg * A + a;
    if (nb >= nblocks) nb = nblocks - 1;
    w[a] = wp + nb * Fmt<F>::kTileQuads + lane;
    s2[a] = row_scale2<F>(scales, nb * 16 + r);
  }
  // X staging: unit q = (row rr = q/32, chunk c = q%32) of the tile; rows
  // beyond M repeat row M-1 (their accumulator columns are never stored).
  const _Float16* xsrc[kPerThread];
  int xdst[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    int q = i * kThreads + tid;
    if (q >= kChunks) q = kChunks - 1;  // surplus threads duplicate the last unit
    const int rr = q >> 5, c = q & 31;
    int64_t m = mg * 16 * MB + rr;
    if (m >= M) m = M - 1;
    xsrc[i] = X + m * K + 8 * c;
    xdst[i] = rr * 32 + (c ^ (rr & 15));
  }
  const int64_t klast = kt1 > kt0 ? kt1 - 1 : kt0;
  auto clampk = [&](int64_t t) { return t < klast ? t : klast; };
  struct XRegs {
    half8v v[kPerThread];
  };
  auto gload_x = [&](XRegs& xr, int64_t kt) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      xr.v[i] = *reinterpret_cast<const half8v*>(xsrc[i] + kt * 256);
  };
  auto swrite_x = [&](const XRegs& xr, int slot) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) xs[slot][xdst[i]] = xr.v[i];
  };

  float4v acc[A * MB];  // row block a, column group b: acc[a * MB + b]
#pragma unroll
  for (int i = 0; i < A * MB; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
  auto load_w = [&](WStage<F, A>& st, int64_t kt) {
#pragma unroll
    for (int a = 0; a < A; ++a) {
      Fmt<F>::template load<MB == 1>(st.t[a], w[a] + kt * kstr, lane);
    }
  };
  auto mac = [&](const WStage<F, A>& st, int slot) {
    const half8v* xb = xs[slot];
#define FP6_XL_STEP(J)                                                                   \
  {                                                                                      \
    half8v bf[MB];                                                                       \
    _Pragma("unroll") for (int b = 0; b < MB; ++b) bf[b] =                               \
        xb[(b * 16 + r) * 32 + ((4 * J + g) ^ r)];                                       \
    _Pragma("unroll") for (int a = 0; a < A; ++a) {                                      \
      const half8v wa = Fmt<F>::template step<J>(st.t[a], s2[a]);                        \
      _Pragma("unroll") for (int b = 0; b < MB; ++b) acc[a * MB + b] =                   \
          __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, bf[b], acc[a * MB + b], 0, 0, 0);   \
    }                                                                                    \
  }
    FP6_XL_STEP(0) FP6_XL_STEP(1) FP6_XL_STEP(2) FP6_XL_STEP(3)
    FP6_XL_STEP(4) FP6_XL_STEP(5) FP6_XL_STEP(6) FP6_XL_STEP(7)
#undef FP6_XL_STEP
  };

  // Tile i of the split (kt = kt0 + i) sits in ring[i % D] and xr[i % D] and
  // is read from LDS slot i % 2.  Iteration i writes X(i+1) into slot
  // (i+1) % 2, whose last reader was iteration i-1 (one barrier between),
  // issues X(i+D) into the freed xr[i % D], consumes ring[i % D], refills it
  // with W(i+D), then meets the barrier.  Branch-free steady state with
  // clamped prefetch indices; the last (< D) tiles run in a tail.
  WStage<F, A> ring[D];
  XRegs xr[D];
  if (kt0 < kt1) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      gload_x(xr[d], clampk(kt0 + d));
      load_w(ring[d], clampk(kt0 + d));
    }
    swrite_x(xr[0], 0);
    __syncthreads();
    int64_t kt = kt0;
    for (; kt + D <= kt1; kt += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int64_t t = kt + d;
        swrite_x(xr[(d + 1) % D], (d + 1) & 1);
        gload_x(xr[d], clampk(t + D));
        mac(ring[d], d & 1);
        load_w(ring[d], clampk(t + D));
        __syncthreads();
      }
    }
#pragma unroll
    for (int d = 0; d + 1 < D; ++d) {
      if (kt + d < kt1) {
        swrite_x(xr[(d + 1) % D], (d + 1) & 1);
        mac(ring[d], d & 1);
        __syncthreads();
      }
    }
  }
  if (!wave_active) return;

  if (splits > 1) {
    const int64_t unit = mg * ngroups + rg;
    float* unit_part = part + unit * static_cast<int64_t>(splits) * (A * MB * 256);
    if (!splitk_fixup<A * MB>(acc, unit_part, counters + unit, split, splits, lane)) return;
  }
#pragma unroll
  for (int a = 0; a < A; ++a) {
    const int64_t nb = rg * A + a;
    if (nb >= nblocks) continue;
#pragma unroll
    for (int b = 0; b < MB; ++b) store_y_block(Y, acc[a * MB + b], (mg * MB + b) * 16 + r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// K-split persistent kernel (memory-bound regime, M <= 16, at most
// kKsWaves*KTW k-tiles per K-split).  One workgroup of kKsWaves (8 or 16)
// waves per CU and K-split.  Wave w owns the k-tiles [w*KT/W, (w+1)*KT/W)
// of its split (W = kKsWaves) for the whole kernel, so its X fragments (16
// columns x at most KTW k-tiles) are staged once, through LDS, into
// registers.  The workgroup walks the row blocks b, b + G, ... (G
// workgroups per split).  With one tile per wave and 2..8 row blocks per
// workgroup (P) the code is straight-line: up to 4 row blocks' tiles in
// flight, every wave multiplies all of its row blocks into partial slots,
// and after one barrier wave i sums row block i; otherwise a loop
// prefetches one row block ahead and wave 0 sums each row block after a
// barrier.  The 16 partial tiles of a row block are summed in wave order
// (deterministic); with K-splits the sum goes through the fixed-order
// split-K fix-up.  No X re-reads, all k-slices of a row block stream
// concurrently.
// ---------------------------------------------------------------------------
template <int F, int KTW, int kKsWaves, bool M1 = false, int P = 0>
__global__ __launch_bounds__(64 * kKsWaves) void fp6_gemm_ksplit(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits) {
  // Per wave, one 8 KB LDS region: first the X staging area of its k-tiles,
  // then (after the wave has read its fragments) its partial-tile buffers of
  // 1 KB each (two, or P).
  __shared__ __attribute__((aligned(16))) half8v xw[kKsWaves][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  // Workgroup b takes K-split b % splits (its k-tiles [kt0, kt1)) of the
  // row blocks b / splits, + gridDim.x / splits, ...  With splits > 1 the
  // summed 16x16 tile of a row block goes through the fixed-order split-K
  // fix-up (the last split to arrive adds the partials in split order).
  const int split = static_cast<int>(blockIdx.x % splits);
  const int64_t kt0 = split * ktiles / splits, kts = (split + 1) * ktiles / splits - kt0;
  const int64_t kw0 = kt0 + wave * kts / kKsWaves, kw1 = kt0 + (wave + 1) * kts / kKsWaves;
  const int ktw = static_cast<int>(kw1 - kw0);  // 0..KTW tiles for this wave
  // Tile indices clamped into the wave's range (or tile 0 for an empty
  // range): clamped slots are loaded but never multiplied.
  auto tile_of = [&](int t) -> int64_t {
    if (ktw == 0) return 0;
    return kw0 + (t < ktw ? t : ktw - 1);
  };
  auto red_at = [&](int buf, int w) { return reinterpret_cast<float4v*>(&xw[w][64 * buf]); };

  // X of this wave's k-slice, loaded coalesced: instruction i covers rows
  // 2i, 2i+1 (512 B each), lane -> 16-byte unit xc of row 2i + lane / 32.  Rows
  // beyond M repeat row M-1 (their accumulator columns are never stored).
  // Fragment loads straight from global memory touch 16 rows per
  // instruction, which costs the L1/L2 path several times the bytes.  With
  // M = 1 all 16 B-operand columns are X's one row: one 8-byte load per lane
  // covers a tile.
  const int xc = lane & 31;
  constexpr int kXLoads = M1 ? 1 : 8;
  half8v xg[KTW][kXLoads];
  [[maybe_unused]] half4v xg1[KTW];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
    if constexpr (M1) {
      xg1[t] = *reinterpret_cast<const half4v*>(X + tile_of(t) * 256 + 4 * lane);
    } else {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int rr = 2 * i + (lane >> 5);
        const int64_t m = rr < M ? rr : M - 1;
        xg[t][i] = *reinterpret_cast<const half8v*>(X + m * K + tile_of(t) * 256 + 8 * xc);
      }
    }
  }
  // Unit (rr, c) is stored at column c ^ rr of row rr, so the 16 lanes of a
  // fragment read (16 rows, same k) hit distinct banks; with M = 1 the row
  // is stored once and every fragment read is a broadcast.  Only this wave
  // touches its region, and a wave's LDS operations complete in order, so
  // a tile's fragments are read before the next tile (or a partial tile)
  // overwrites them, with no barrier.
  half8v xf[KTW][8];
  auto stage_x = [&]() {
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      if constexpr (M1) {
        reinterpret_cast<half4v*>(&xw[wave][0])[lane] = xg1[t];
#pragma unroll
        for (int j = 0; j < 8; ++j) xf[t][j] = xw[wave][4 * j + g];
      } else {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
          const int rr = 2 * i + (lane >> 5);
          xw[wave][rr * 32 + (xc ^ rr)] = xg[t][i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xf[t][j] = xw[wave][r * 32 + ((4 * j + g) ^ r)];
      }
    }
  };

  // A row block's tiles and its row scale travel together: vector loads
  // complete in issue order, so a scale requested after the next row
  // block's tiles would make this one wait for them.
  WStage<F, 1> wst[2][KTW];
  _Float16 wsc[2];
  auto load_rb = [&](WStage<F, 1> (&st)[KTW], _Float16& sc, int64_t nb) {
    const u32x4* base = wp + nb * Fmt<F>::kTileQuads + lane;
#pragma unroll
    for (int t = 0; t < KTW; ++t) Fmt<F>::template load<true>(st[t].t[0], base + tile_of(t) * kstr, lane);
    sc = scales[nb * 16 + r];
  };
  auto rb_mac = [&](const WStage<F, 1> (&st)[KTW], _Float16 sc) {
    const half2v s2 = scale2_of<F>(sc);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    // With one tile per wave the products run unconditionally and an empty
    // k-range (tile 0 loaded as a stand-in) is zeroed afterwards: behind a
    // branch the compiler sinks a row block's loads into it, past earlier
    // waits.
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      if (KTW == 1 || t < ktw) {
#define FP6_KS_STEP(J)                                                                     \
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(                                            \
      Fmt<F>::template step<J>(st[t].t[0], s2), xf[t][J], acc, 0, 0, 0);
        FP6_KS_STEP(0) FP6_KS_STEP(1) FP6_KS_STEP(2) FP6_KS_STEP(3)
        FP6_KS_STEP(4) FP6_KS_STEP(5) FP6_KS_STEP(6) FP6_KS_STEP(7)
#undef FP6_KS_STEP
      }
    }
    if (KTW == 1 && ktw == 0) acc = float4v{0.f, 0.f, 0.f, 0.f};
    return acc;
  };
  // Row block nb's summed tile: stored, or (with K-splits) handed to the
  // fix-up, whose last arriver stores.
  auto finish = [&](float4v sum, int64_t nb) {
    if (splits > 1) {
      float4v a1[1] = {sum};
      if (!splitk_fixup<1>(a1, part + nb * splits * 256, counters + nb, split, splits, lane)) return;
      sum = a1[0];
    }
    store_y_block(Y, sum, r, M, N, nb * 16, g);
  };
  auto reduce_store = [&](const float4v& acc, int buf, int64_t nb) {
    red_at(buf, wave)[lane] = acc;
    __syncthreads();
    // A plain loop: this kernel keeps the next row block's tiles and its X
    // slice in registers, so holding several partial tiles at once spills.
    if (wave == 0) {
      float4v sum = red_at(buf, 0)[lane];
#pragma unroll
      for (int w = 1; w < kKsWaves; ++w) sum += red_at(buf, w)[lane];
      finish(sum, nb);
    }
  };

  const int64_t stride = gridDim.x / splits;
  int64_t nb = blockIdx.x / splits;
  if (nb >= nblocks) return;  // uniform for the workgroup
  if constexpr (P > 0) {
    static_assert(P <= 8 && P <= kKsWaves, "P partial tiles per wave region, one summing wave each");
    // At most P row blocks per workgroup, held in S register stages: the
    // first S are requested at once, and row block i + S into stage i % S
    // right after row block i's products.  Straight-line code: a workgroup
    // with fewer row blocks repeats its last one (loads, products and the
    // store of identical values) instead of branching, since behind a
    // branch the compiler sinks the loads past the X staging's wait and
    // the waits after it then cover every row block.
    constexpr int S = P < 4 ? P : 4;
    WStage<F, 1> ast[S][KTW];
    _Float16 asc[S];
    const int64_t nlast = nb + ((nblocks - 1 - nb) / stride) * stride;
    auto rb_of = [&](int i) {
      const int64_t nbi = nb + i * stride;
      return nbi < nlast ? nbi : nlast;
    };
#pragma unroll
    for (int i = 0; i < S; ++i) load_rb(ast[i], asc[i], rb_of(i));
    // Fence: left free, the scheduler moves the last row scales down into
    // the first row block's products, after its waits.
    __builtin_amdgcn_sched_barrier(0);
    stage_x();
    // Every wave multiplies all of its row blocks into its partial-tile
    // slots before the one barrier, so a wave whose tiles have arrived does
    // not wait for the slowest wave of each row block in turn.  Wave i then
    // sums and stores row block i.
#pragma unroll
    for (int i = 0; i < P; ++i) {
      red_at(i, wave)[lane] = rb_mac(ast[i % S], asc[i % S]);
      if (i + S < P) load_rb(ast[i % S], asc[i % S], rb_of(i + S));
    }
    __syncthreads();
    if (wave < P && nb + wave * stride <= nlast) {  // repeated row blocks are not stored again
      float4v sum = red_at(wave, 0)[lane];
#pragma unroll
      for (int w = 1; w < kKsWaves; ++w) sum += red_at(wave, w)[lane];
      finish(sum, nb + wave * stride);
    }
    return;
  }
  // The first two row blocks' tiles are requested before X is staged (whose
  // LDS writes wait for the X loads, issued first).
  int64_t nb1 = nb + stride;
  load_rb(wst[0], wsc[0], nb);
  load_rb(wst[1], wsc[1], nb1 < nblocks ? nb1 : nb);
  stage_x();
  // Two row blocks per iteration so the register double buffer is static.
  // The partial-tile buffers alternate too: a buffer is rewritten only after
  // the next barrier, by which time wave 0 has finished reading it.
  while (true) {
    reduce_store(rb_mac(wst[0], wsc[0]), 0, nb);
    if (nb1 >= nblocks) break;
    const int64_t nb2 = nb1 + stride;
    load_rb(wst[0], wsc[0], nb2 < nblocks ? nb2 : nb1);
    reduce_store(rb_mac(wst[1], wsc[1]), 1, nb1);
    if (nb2 >= nblocks) break;
    nb = nb2;
    nb1 = nb + stride;
    load_rb(wst[1], wsc[1], nb1 < nblocks ? nb1 : nb);
  }
}

// ---------------------------------------------------------------------------
// K-ring kernel (memory-bound regime, M <= 16, K <= 8192, at most 8 row
// blocks per CU).  One 8-wave workgroup per CU owns P consecutive row blocks
// (P = row blocks over CUs, rounded up) over the whole K range.  Wave w owns
// the k-tiles [w*KT/8, (w+1)*KT/8) (at most KTW) and keeps their X fragments
// in registers for the whole kernel, so the loop has no X staging, no LDS
// read and no barrier.  The wave walks the workgroup's row blocks in order
// through a register ring of KTW tiles: the next row block's tile t is
// requested as soon as this row block's tile t has been multiplied, and its
// row scale right after its first tile.  Each row block's partial tile goes
// to the wave's LDS region; after one barrier wave i sums row block i over
// the 8 waves in wave order (deterministic).  When the row blocks divide
// evenly over the CUs (Llama-70B MLP: 1792 = 7 x 256) every SIMD streams the
// same number of tiles.  Tiles beyond a wave's range (K/256 not a multiple
// of 8) are loaded as stand-ins and multiplied by zero X fragments.  With
// M = 1 (M1) all 16 B-operand columns are X's one row: each lane loads its
// fragments directly (16 bytes per k-step, 64 distinct bytes per wave
// instruction), with no staging.  With K split across workgroups (splits >
// 1, for K > 8192) workgroup b runs split b % splits of row group b /
// splits, and the summed tile of a row block goes through the fixed-order
// split-K fix-up.  R row blocks are in flight per wave (ring slot sets).
// ---------------------------------------------------------------------------
template <int F, int KTW, bool M1 = false, int R = 1>
__global__ __launch_bounds__(512) void fp6_gemm_kring(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int P, int splits) {
  constexpr int kWaves = 8;
  // Per wave 8 KB: first the X staging area of one k-tile (16 rows x 512 B),
  // then the partial tiles of its row blocks (1 KB each, P <= 8).
  __shared__ __attribute__((aligned(16))) half8v xw[kWaves][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int split = static_cast<int>(umod32(blockIdx.x, splits));
  const int64_t kt0 = split * ktiles / splits, kts = (split + 1) * ktiles / splits - kt0;
  const int64_t kw0 = kt0 + wave * kts / kWaves, kw1 = kt0 + (wave + 1) * kts / kWaves;
  const int ktw = static_cast<int>(kw1 - kw0);  // 0..KTW tiles for this wave
  const int64_t nb0 = static_cast<int64_t>(udiv32(blockIdx.x, splits)) * P;
  if (nb0 >= nblocks) return;  // uniform for the workgroup
  const int pw = static_cast<int>(nblocks - nb0 < P ? nblocks - nb0 : P);
  auto tile_of = [&](int t) -> int64_t {
    if (ktw == 0) return 0;
    return kw0 + (t < ktw ? t : ktw - 1);
  };

  // X of this wave's k-tiles, loaded coalesced first (instruction i covers
  // rows 2i, 2i+1, lane -> 16-byte unit xc of row 2i + lane/32; rows beyond
  // M repeat row M-1, whose accumulator columns are never stored).
  const int xc = lane & 31;
  half8v xg[KTW][8];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (M1) {
        xg[t][i] = *reinterpret_cast<const half8v*>(X + tile_of(t) * 256 + 32 * i + 8 * g);
      } else {
        const int rr = 2 * i + (lane >> 5);
        const int64_t m = rr < M ? rr : M - 1;
        xg[t][i] = *reinterpret_cast<const half8v*>(X + m * K + tile_of(t) * 256 + 8 * xc);
      }
    }
  }
  // The first row block's tiles with its row scale after the first tile:
  // the order the loop below issues the next row block's loads in, so that
  // the compiler's wait counts at the loop head are exact.
  // R row blocks in flight: ring slot set rr holds row blocks rr, rr + R,
  // ...  Requests past the last row block repeat it (cache hits).
  WStage<F, 1> ring[R][KTW];
  const int64_t nb_last = nb0 + pw - 1;
  auto tile_ptr = [&](int64_t nb, int t) { return wp + nb * Fmt<F>::kTileQuads + lane + tile_of(t) * kstr; };
  _Float16 sc[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int64_t nb = nb0 + rr < nb_last ? nb0 + rr : nb_last;
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      Fmt<F>::template load<true>(ring[rr][t].t[0], tile_ptr(nb, t), lane);
      if (t == 0) sc[rr] = scales[nb * 16 + r];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Stage X through the wave's LDS region into B fragments: unit (rr, c) at
  // column c ^ rr of row rr, so the 16 lanes of a fragment read hit distinct
  // banks.  Only this wave uses its region and its LDS operations complete in
  // order, so no barrier is needed between tiles.
  half8v xf[KTW][8];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
    const bool live = t < ktw;
    if constexpr (M1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xf[t][j] = live ? xg[t][j] : half8v{};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 2 * i + (lane >> 5);
        xw[wave][rr * 32 + (xc ^ rr)] = xg[t][i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half8v v = xw[wave][r * 32 + ((4 * j + g) ^ r)];
        xf[t][j] = live ? v : half8v{};
      }
    }
  }

  // Row block i: its tiles are in ring slot set SLOT; as tile t is
  // multiplied, the slot is refilled with tile t of row block i + R (NEXT),
  // and its row scale is requested after its first tile.
  auto row_block = [&](int i, auto SLOT, auto NEXT) {
    constexpr int kSlot = decltype(SLOT)::value;
    constexpr bool kNext = decltype(NEXT)::value;
    const half2v s2 = scale2_of<F>(sc[kSlot]);
    const int64_t nbn = nb0 + i + R < nb_last ? nb0 + i + R : nb_last;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
#define FP6_KR_STEP(J)                                                                             \
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<J>(ring[kSlot][t].t[0], s2), \
                                               xf[t][J], acc, 0, 0, 0);
      FP6_KR_STEP(0) FP6_KR_STEP(1) FP6_KR_STEP(2) FP6_KR_STEP(3)
      FP6_KR_STEP(4) FP6_KR_STEP(5) FP6_KR_STEP(6) FP6_KR_STEP(7)
#undef FP6_KR_STEP
      if constexpr (kNext) {
        // Fences: left free, the scheduler sinks these loads to the end of
        // the row block, so the ring would refill a row block at a time.
        __builtin_amdgcn_sched_barrier(0);
        Fmt<F>::template load<true>(ring[kSlot][t].t[0], tile_ptr(nbn, t), lane);
        if (t == 0) sc[kSlot] = scales[nbn * 16 + r];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    reinterpret_cast<float4v*>(&xw[wave][64 * i])[lane] = acc;
  };
  // Groups of R row blocks while a successor exists, then a tail of at most
  // R row blocks that requests nothing.
  int i = 0;
  for (; i + R < pw; i += R) {
    row_block(i, std::integral_constant<int, 0>{}, std::true_type{});
    if constexpr (R > 1) row_block(i + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  row_block(i, std::integral_constant<int, 0>{}, std::false_type{});
  if constexpr (R > 1) {
    if (i + 1 < pw) row_block(i + 1, std::integral_constant<int, 1>{}, std::false_type{});
  }
  __syncthreads();
  if (wave < pw) {
    const int64_t nb = nb0 + wave;
    float4v sum[1] = {reinterpret_cast<const float4v*>(&xw[0][64 * wave])[lane]};
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum[0] += reinterpret_cast<const float4v*>(&xw[w][64 * wave])[lane];
    if (splits > 1 && !splitk_fixup<1>(sum, part + nb * splits * 256, counters + nb, split, splits, lane))
      return;
    store_y_block(Y, sum[0], r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// K-slice kernel (memory-bound regime, M <= 16, few row blocks, long K).
// Like the k-split kernel, WK waves of a workgroup split the K range of a row
// block and reduce through LDS, but each wave issues the loads of all its
// packed tiles at once and streams its X fragments half-tile by half-tile
// (a ring of three, two ahead) instead of keeping them resident.  One
// workgroup per row block: meant for N/16 <= CUs, where X is used once per CU
// anyway.
// ---------------------------------------------------------------------------
template <int F, int KTW, int WK, bool M1 = false>
__global__ __launch_bounds__(64 * WK) void fp6_gemm_kslice(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, int64_t M, int64_t N,
    int64_t K) {
  __shared__ float4v red[WK][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int64_t kw0 = wave * ktiles / WK, kw1 = (wave + 1) * ktiles / WK;
  const int ktw = static_cast<int>(kw1 - kw0);
  auto tile_of = [&](int t) -> int64_t {
    if (ktw == 0) return 0;
    return kw0 + (t < ktw ? t : ktw - 1);
  };
  const int64_t m = r < M ? r : M - 1;
  const _Float16* xrow = X + m * K + 8 * g;
  // X fragments stream through a ring of 3 half-tiles (4 k-steps each),
  // loaded two half-tiles ahead of their use.
  auto load_xh = [&](half8v (&xf)[4], int hh) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xf[j] = *reinterpret_cast<const half8v*>(xrow + tile_of(hh >> 1) * 256 + 128 * (hh & 1) + 32 * j);
  };

  {
    // One row block per workgroup (the grid has one workgroup per row
    // block).  With a loop over row blocks the compiler would hoist the X
    // loads (they do not depend on the row block) and keep them all live.
    const int64_t nb = blockIdx.x;
    if (nb >= nblocks) return;  // uniform for the workgroup
    const u32x4* base = wp + nb * Fmt<F>::kTileQuads + lane;
    // M = 1 (KTW = 1): the 16 columns of the B operand all repeat X's single
    // row, so each lane loads just 8 of the tile's 256 values (one 8-byte
    // load, issued before the weights so that waiting for it does not wait
    // for them) into the wave's own LDS slice and reads its fragments back
    // from there (one address per lane group: an LDS broadcast).  A wave only
    // reads its own slice, and LDS operations of a wave complete in order,
    // so no barrier is needed.
    [[maybe_unused]] half4v x1 = {};
    if constexpr (M1) x1 = *reinterpret_cast<const half4v*>(X + tile_of(0) * 256 + 4 * lane);
    WStage<F, 1> st[KTW];
#pragma unroll
    for (int t = 0; t < KTW; ++t) Fmt<F>::template load<true>(st[t].t[0], base + tile_of(t) * kstr, lane);
    const half2v s2 = row_scale2<F>(scales, nb * 16 + r);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KTW == 1) {
      // One tile per wave: all of its X fragments are loaded at once.
      half8v xf[8];
      if constexpr (M1) {
        static_assert(KTW == 1, "the M = 1 staging covers one tile per wave");
        __shared__ half8v xw[WK][32];
        reinterpret_cast<half4v*>(&xw[wave][0])[lane] = x1;
#pragma unroll
        for (int j = 0; j < 8; ++j) xf[j] = xw[wave][4 * j + g];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xf[j] = *reinterpret_cast<const half8v*>(xrow + tile_of(0) * 256 + 32 * j);
      }
      // With M1 the MFMAs run unconditionally and an empty k-range (ktw = 0,
      // tile 0 loaded as a stand-in) is zeroed afterwards: behind a branch
      // the compiler would sink the weight loads into it, after the X
      // staging's wait.
      if (M1 || ktw > 0) {
        // Two accumulators halve the MFMA dependency chain.
        float4v acc1 = {0.f, 0.f, 0.f, 0.f};
#define FP6_KX1(J, A)                                                                       \
  A = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<J>(st[0].t[0], s2), xf[J], A, 0, 0, 0);
        FP6_KX1(0, acc) FP6_KX1(1, acc1) FP6_KX1(2, acc) FP6_KX1(3, acc1)
        FP6_KX1(4, acc) FP6_KX1(5, acc1) FP6_KX1(6, acc) FP6_KX1(7, acc1)
#undef FP6_KX1
        acc += acc1;
        if (M1 && ktw == 0) acc = float4v{0.f, 0.f, 0.f, 0.f};
      }
    } else {
    half8v xr[3][4];
    load_xh(xr[0], 0);
    load_xh(xr[1], 1);
#pragma unroll
    for (int hh = 0; hh < 2 * KTW; ++hh) {
      if (hh + 2 < 2 * KTW) load_xh(xr[(hh + 2) % 3], hh + 2);
      const int t = hh >> 1;
      if (t < ktw) {
        const half8v* xf = xr[hh % 3];
        if (hh & 1) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<4>(st[t].t[0], s2), xf[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<5>(st[t].t[0], s2), xf[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<6>(st[t].t[0], s2), xf[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<7>(st[t].t[0], s2), xf[3], acc, 0, 0, 0);
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<0>(st[t].t[0], s2), xf[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<1>(st[t].t[0], s2), xf[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<2>(st[t].t[0], s2), xf[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Fmt<F>::template step<3>(st[t].t[0], s2), xf[3], acc, 0, 0, 0);
        }
      }
      // Keep the X prefetch two half-tiles ahead: without this fence the
      // scheduler hoists every half-tile's X loads to the top and runs out of
      // registers.
      __builtin_amdgcn_sched_barrier(0);
    }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) store_y_block(Y, reduce_waves<WK>(red, lane), r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// Tiled fused kernel (compute-bound regime, M > 16).
// Workgroup = 4 waves; tile = 256 weight rows (each wave 4 row blocks = 64
// rows) x BM = 16*B columns of X.  Every weight is spliced once per
// workgroup and reused for B MFMAs; every X fragment (16 columns x 32 k) is
// read from LDS and reused for the wave's 4 row blocks.
// Pipeline per half-tile h (128 k = 4 k-steps):
//   * X(h+1) is copied global -> LDS by direct LDS loads (no registers) into
//     the buffer freed by the previous barrier; rows are XOR-swizzled in
//     16-byte units (on the global side, since the LDS side of a direct load
//     is linear) so the B-fragment reads are free of bank conflicts;
//   * the packed weight words of half-tile h+1 are loaded into registers;
//   * the 4*B MFMAs of k-step J run while the A fragments of k-step J+1 are
//     spliced and its B fragments read (sched_group_barrier interleaves one
//     MFMA with three VALU ops);
//   * each wave waits for its own direct loads, then one barrier.
// ---------------------------------------------------------------------------

// Workgroup barrier without the release fence of __syncthreads().  The
// fence makes a wave wait for every direct LDS load it has in flight, so a
// copy issued several stages ahead would be waited for at once; the callers
// instead wait (s_waitcnt) for exactly the copies the next stage reads.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup index -> logical tile index, XCD-aware.  Workgroups are handed
// to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), each XCD with
// its own L2.  This gives XCD x the contiguous logical range
// [x*q + min(x, r), ...) (q = G/8, r = G%8, the first r XCDs one more), so
// workgroups that share operands (the K-splits of a row tile, the row tiles
// of one column group and their X slice) meet in the same L2.  A bijection
// on [0, G).
__device__ __forceinline__ int64_t xcd_logical_block(int64_t b, int64_t G) {
  constexpr int kXcds = 8;
  const int64_t x = b % kXcds, j = b / kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + j;
}

template <int F, int TA>
struct WHalf {           // packed words of one half-tile for TA row blocks
  typename Fmt<F>::Half h[TA];
};

template <int F, int JJ, int TA>
__device__ __forceinline__ void splice_half(half8v (&dst)[TA], const WHalf<F, TA>& w, const half2v (&s2)[TA]) {
#pragma unroll
  for (int a = 0; a < TA; ++a) dst[a] = Fmt<F>::template half_step<JJ>(w.h[a], s2[a]);
}

// One workgroup's pass over half-tiles [h0, h1) of its tile (m-group mg,
// 256-row tile nt), accumulated into acc.  X half-tiles go through the LDS
// buffers xbuf0/xbuf1 (distinct __shared__ arrays of the caller).
template <int F, int B, int TA, int NW>
__device__ __forceinline__ void tiled_run(const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
                                          const _Float16* __restrict__ scales, int64_t M, int64_t N,
                                          int64_t K, int64_t mg, int64_t nt, int64_t h0, int64_t h1,
                                          half8v* xbuf0, half8v* xbuf1, float4v (&acc)[TA * B]) {
  constexpr int BM = 16 * B;
  constexpr int kHalfUnits = BM * 16;             // 16-byte units per X half-tile buffer
  constexpr int kTA = TA;
  constexpr int kThreads = 64 * NW;
  static_assert(TA * NW == 16, "a workgroup covers 16 row blocks");
  constexpr int kLoadsPerThread = kHalfUnits / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = mg * BM;

  // Weights: this wave's TA row blocks (ragged N: repeat the last block).
  // The row scales are loaded after the first tile's loads are in flight.
  const u32x4* w[kTA];
  int64_t srow[kTA];
  half2v s2[kTA];
#pragma unroll
  for (int a = 0; a < kTA; ++a) {
    int64_t nb = nt * 16 + wave * kTA + a;
    if (nb >= nblocks) nb = nblocks - 1;
    w[a] = wp + nb * Fmt<F>::kTileQuads + lane;
    srow[a] = nb * 16 + r;
  }
  auto load_wh = [&](WHalf<F, TA>& st, int64_t h) {  // half-tile h: k-tile h>>1, half h&1
    const int64_t kt = h >> 1;
    const int hh = static_cast<int>(h & 1);
#pragma unroll
    for (int a = 0; a < kTA; ++a) {
      Fmt<F>::load_half(st.h[a], w[a] + kt * kstr, hh, lane);
    }
  };

  // X direct loads: instruction i of this wave fills LDS units
  // [i*kThreads + wave*64, +64) linearly; unit u = (row mm = u/16, slot
  // c' = u%16) receives global chunk c = c' ^ (mm & 15) of X row m0+mm.
  const _Float16* xsrc[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int u = i * kThreads + tid, mm = u >> 4, c = (u & 15) ^ (mm & 15);
    int64_t m = m0 + mm;
    if (m >= M) m = M - 1;
    xsrc[i] = X + m * K + 8 * c;
  }
  auto dma_x = [&](half8v* buf, int64_t h) {
    const int64_t koff = (h >> 1) * 256 + (h & 1) * 128;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(xsrc[i] + koff),
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(buf + i * kThreads + wave * 64)),
          16, 0, 0);
  };

  half8v afr[2][kTA];
  half8v bfr[2][B];
  auto read_b = [&](half8v (&bf)[B], const half8v* buf, int jj) {
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const int mm = bi * 16 + r, c = 4 * jj + g;
      bf[bi] = buf[mm * 16 + (c ^ (mm & 15))];
    }
  };
  auto mfmas = [&](const half8v (&av)[kTA], const half8v (&bf)[B]) {
#pragma unroll
    for (int a = 0; a < kTA; ++a)
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
        acc[a * B + bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bf[bi], acc[a * B + bi], 0, 0, 0);
  };
  // Per k-step: 1 MFMA then 3 VALU (the next splice), with the B-fragment
  // reads of the next k-step placed after the first 2 MFMAs.  The reads of
  // the k-step being multiplied were issued one k-step earlier, so the wait
  // before its first MFMA finds them done; issued ahead of those MFMAs
  // instead, 16 reads would be in flight, more than the LDS counter can
  // track, and the compiler then waits for all of them.
  auto interleave = [&](auto NDS) {
    constexpr int nds = decltype(NDS)::value;
#pragma unroll
    for (int i = 0; i < kTA * B; ++i) {
      if constexpr (nds > 0) {
        if (i == 2) __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using IB = std::integral_constant<int, B>;
  // Wait for this wave's direct LDS loads of the next half-tile (issued
  // before the kTA*2 weight loads of that half-tile), then the barrier makes
  // every wave's copy visible.
  constexpr int kWLoads = kTA * Fmt<F>::kHalfLoads;
  constexpr int kWaitDma = (kWLoads & 15) | ((kWLoads >> 4) << 14) | (7 << 4) | (15 << 8);

  // One half-tile: k-steps 0..3 from buffer `cur`; prefetch X(h+1) into
  // `nxt` and the weights of h+1 into `wn`; overlap the last k-step with the
  // splice of h+1's first k-step.
  auto half_step = [&](half8v* cur, half8v* nxt, const WHalf<F, TA>& wc, WHalf<F, TA>& wn, int64_t hnext) {
    dma_x(nxt, hnext);
    __builtin_amdgcn_sched_barrier(0);
    load_wh(wn, hnext);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[0], cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[1], cur, 1); splice_half<F, 1, TA>(afr[1], wc, s2); mfmas(afr[0], bfr[0]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[0], cur, 2); splice_half<F, 2, TA>(afr[0], wc, s2); mfmas(afr[1], bfr[1]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[1], cur, 3); splice_half<F, 3, TA>(afr[1], wc, s2); mfmas(afr[0], bfr[0]); interleave(IB{});
    // Fence: the splice below reads the words of h+1, just requested; left
    // free, the scheduler pulls it into the first k-step's VALU slots and the
    // wave waits for those loads there (measured: 2.5-4% at M >= 128).
    __builtin_amdgcn_sched_barrier(0);
                            splice_half<F, 0, TA>(afr[0], wn, s2); mfmas(afr[1], bfr[1]); interleave(I0{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitDma);
    __syncthreads();
  };

  if (h0 < h1) {
    // Branch-free steady state: prefetch indices are clamped to the split's
    // last half-tile, so every path has the same loads in flight.
    auto clamph = [&](int64_t h) { return h < h1 - 1 ? h : h1 - 1; };
    // One round trip: the first half-tile's X and words, then the row
    // scales, all in flight together; the fences keep the compiler from
    // starting the first splice (which waits for the words) between them.
    WHalf<F, TA> wa, wb;
    dma_x(xbuf0, h0);
    load_wh(wa, h0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int a = 0; a < kTA; ++a) s2[a] = row_scale2<F>(scales, srow[a]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    splice_half<F, 0, TA>(afr[0], wa, s2);
    int64_t h = h0;
    for (; h + 2 <= h1; h += 2) {
      half_step(xbuf0, xbuf1, wa, wb, clamph(h + 1));
      half_step(xbuf1, xbuf0, wb, wa, clamph(h + 2));
    }
    if (h < h1) half_step(xbuf0, xbuf1, wa, wb, clamph(h + 1));  // odd count (stream-K segments)
  }

}

// Store a tiled workgroup's accumulators (rows of row tile nt, columns of
// m-group mg); ragged N: the repeated last row block is not stored.
template <int B, int TA>
__device__ __forceinline__ void tiled_store(_Float16* __restrict__ Y, const float4v (&acc)[TA * B], int64_t M,
                                            int64_t N, int64_t mg, int64_t nt, int wave, int lane) {
  const int64_t nblocks = N >> 4;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    const int64_t nb = nt * 16 + wave * TA + a;
    if (nb >= nblocks) continue;
#pragma unroll
    for (int bi = 0; bi < B; ++bi)
      store_y_block(Y, acc[a * B + bi], mg * 16 * B + bi * 16 + r, M, N, nb * 16, g);
  }
}

// TA row blocks per wave, NW waves per workgroup, TA * NW = 16 (256 rows).
// Split-K: workgroup (tile, split) runs the split's k-tiles.
template <int F, int B, int TA, int NW>
__global__ __launch_bounds__(64 * NW) void fp6_gemm_tiled(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  constexpr int kHalfUnits = 16 * B * 16;
  __shared__ __attribute__((aligned(16))) half8v xbuf0[kHalfUnits];
  __shared__ __attribute__((aligned(16))) half8v xbuf1[kHalfUnits];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t ntiles = (nblocks + 15) >> 4;     // 256-row workgroup tiles
  const uint32_t lb = static_cast<uint32_t>(xcd_logical_block(blockIdx.x, gridDim.x));
  const int split = static_cast<int>(umod32(lb, splits));
  const uint32_t bidx = udiv32(lb, splits);
  const uint32_t bq = udiv32(bidx, static_cast<uint32_t>(ntiles));
  const int64_t nt = bidx - bq * static_cast<uint32_t>(ntiles);
  const int64_t mg = bq + mg_base;
  const int64_t kt0 = udiv32(split * static_cast<uint32_t>(ktiles), splits);
  const int64_t kt1 = udiv32((split + 1) * static_cast<uint32_t>(ktiles), splits);

  float4v acc[TA * B];
#pragma unroll
  for (int i = 0; i < TA * B; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
  tiled_run<F, B, TA, NW>(X, wp, scales, M, N, K, mg, nt, 2 * kt0, 2 * kt1, xbuf0, xbuf1, acc);

  if (splits > 1) {
    const int64_t unit = (mg * ntiles + nt) * NW + wave;
    float* unit_part = part + unit * static_cast<int64_t>(splits) * (TA * B * 256);
    if (!splitk_fixup<TA * B, true>(acc, unit_part, counters + unit, split, splits, lane)) return;
  }
  tiled_store<B, TA>(Y, acc, M, N, mg, nt, wave, lane);
}

// Stream-K form: the G workgroups (one per CU) split the launch's
// (tile, half-tile) units into G contiguous, equal ranges in tile-major
// order, so every CU does the same number of half-tiles (+-1) whatever the
// tile count.  A range covers the tail of one tile, whole tiles and the head
// of another; each piece is run as one segment.  A tile's pieces come from
// workgroups wf..wl (computable from the range bounds) and meet in the
// fixed-order fix-up (piece order = workgroup order), whose partials sit in
// slots [wf + tile, wf + tile + pieces) of the workspace (disjoint between
// tiles, G + tiles slots of NW waves each).  Workgroups process their range
// in order, so a tile's head piece, run last by its workgroup, is usually
// the last to arrive: the probe-first fix-up lets it sum without a store.
template <int F, int B, int TA, int NW>
__global__ __launch_bounds__(64 * NW) void fp6_gemm_tiled_sk(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int, int64_t) {
  constexpr int kHalfUnits = 16 * B * 16;
  constexpr int kAcc = TA * B;
  __shared__ __attribute__((aligned(16))) half8v xbuf0[kHalfUnits];
  __shared__ __attribute__((aligned(16))) half8v xbuf1[kHalfUnits];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t w = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t nblocks = N >> 4, htiles = 2 * (K >> 8);
  const int64_t ntiles = (nblocks + 15) >> 4;
  const int64_t tiles = ((M + 16 * B - 1) / (16 * B)) * ntiles;
  const int64_t T = tiles * htiles;
  // With fewer units than workgroups, only the first T take part (one unit
  // each): every range is then non-empty, so each workgroup that a tile's
  // range bounds cover does arrive at its fix-up.
  const int64_t G = T < static_cast<int64_t>(gridDim.x) ? T : static_cast<int64_t>(gridDim.x);
  if (w >= G) return;
  int64_t u = w * T / G;
  const int64_t u1 = (w + 1) * T / G;
  while (u < u1) {
    const int64_t tile = u / htiles, hs = u - tile * htiles;
    const int64_t he = (u1 - u < htiles - hs) ? hs + (u1 - u) : htiles;
    const int64_t mg = tile / ntiles, nt = tile - mg * ntiles;
    float4v acc[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
    tiled_run<F, B, TA, NW>(X, wp, scales, M, N, K, mg, nt, hs, he, xbuf0, xbuf1, acc);
    // Workgroups holding the tile's first and last units.
    const int64_t wf = ((tile * htiles + 1) * G - 1) / T;
    const int64_t wl = ((tile + 1) * htiles * G - 1) / T;
    bool finish = true;
    if (wl > wf) {
      float* unit_part = part + ((wf + tile) * NW + wave) * (kAcc * 256);
      finish = splitk_fixup<kAcc, true>(acc, unit_part, counters + tile * NW + wave, static_cast<int>(w - wf),
                                         static_cast<int>(wl - wf + 1), lane, NW * kAcc * 64);
    }
    if (finish) tiled_store<B, TA>(Y, acc, M, N, mg, nt, wave, lane);
    u = tile * htiles + he;
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel with the packed weights staged in LDS (compute-bound regime,
// M > 64).  Same tile and MFMA schedule as fp6_gemm_tiled (NW waves x TA
// row blocks = 256 rows, BM = 16*B columns, half-tile steps), but every
// global load is a direct LDS load: X(h+1) into a two-stage ring shared by
// the workgroup, and each wave's own packed words of half-tile h+3 into a
// four-stage ring, so the weights (from HBM) have three half-tiles of
// compute to arrive and X (from L2) one.  A wave reads its words back from
// LDS one half-tile before it splices them.  The waits are explicit vmcnt
// counts (every load in flight is a direct LDS load, issued in a fixed
// order), and the barrier carries no release fence, which would wait for
// every copy in flight.  Each ring stage is its own LDS array so that the
// compiler, too, tells the copies into one stage from the reads of another.
// ---------------------------------------------------------------------------
template <int F, int TA>
struct WHalfL {
  typename Fmt<F>::Half h[TA];
};

template <int F, int B, int TA, int NW>
__global__ __launch_bounds__(64 * NW) void fp6_gemm_tiledl(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  constexpr int BM = 16 * B;
  constexpr int kHalfUnits = BM * 16;             // 16-byte units per X half-tile stage
  constexpr int kThreads = 64 * NW;
  static_assert(TA * NW == 16, "a workgroup covers 16 row blocks");
  constexpr int kLoadsPerThread = kHalfUnits / kThreads;
  constexpr int kStage = Fmt<F>::kStageBytes;
  constexpr int kWUnits = 16 * kStage / 16;       // 16-byte units per weight stage
  __shared__ __attribute__((aligned(16))) half8v xb0[kHalfUnits];
  __shared__ __attribute__((aligned(16))) half8v xb1[kHalfUnits];
  __shared__ __attribute__((aligned(16))) u32x4 wl0[kWUnits];
  __shared__ __attribute__((aligned(16))) u32x4 wl1[kWUnits];
  __shared__ __attribute__((aligned(16))) u32x4 wl2[kWUnits];
  __shared__ __attribute__((aligned(16))) u32x4 wl3[kWUnits];

  // The wave index is uniform: kept in a scalar register, the LDS addresses
  // of the direct loads need no per-load conversion.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int64_t ntiles = (nblocks + 15) >> 4;     // 256-row workgroup tiles
  const uint32_t lb = static_cast<uint32_t>(xcd_logical_block(blockIdx.x, gridDim.x));
  const int split = static_cast<int>(umod32(lb, splits));
  const uint32_t bidx = udiv32(lb, splits);
  const uint32_t bq = udiv32(bidx, static_cast<uint32_t>(ntiles));
  const int64_t nt = bidx - bq * static_cast<uint32_t>(ntiles);
  const int64_t mg = bq + mg_base;
  const int64_t kt0 = udiv32(split * static_cast<uint32_t>(ktiles), splits);
  const int64_t kt1 = udiv32((split + 1) * static_cast<uint32_t>(ktiles), splits);
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = mg * BM;

  // Weights: this wave's TA row blocks (ragged N: repeat the last block).
  const u32x4* w[TA];
  half2v s2[TA];
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    int64_t nb = nt * 16 + wave * TA + a;
    if (nb >= nblocks) nb = nblocks - 1;
    w[a] = wp + nb * Fmt<F>::kTileQuads + lane;
    s2[a] = row_scale2<F>(scales, nb * 16 + r);
  }
  // This wave's row block a in a weight stage.
  auto wregion = [&](u32x4* stage, int a) { return reinterpret_cast<char*>(stage) + (wave * TA + a) * kStage; };
  auto stage_w = [&](u32x4* stage, int64_t h) {
    const int64_t kt = h >> 1;
    const int hh = static_cast<int>(h & 1);
#pragma unroll
    for (int a = 0; a < TA; ++a) Fmt<F>::stage_half(wregion(stage, a), w[a] + kt * kstr, hh, lane);
  };
  auto read_w = [&](WHalfL<F, TA>& st, u32x4* stage) {
#pragma unroll
    for (int a = 0; a < TA; ++a) Fmt<F>::read_half(st.h[a], wregion(stage, a), lane);
  };

  // X direct loads as in fp6_gemm_tiled (16-byte units XOR-swizzled per row).
  const _Float16* xsrc[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int u = i * kThreads + tid, mm = u >> 4, c = (u & 15) ^ (mm & 15);
    int64_t m = m0 + mm;
    if (m >= M) m = M - 1;
    xsrc[i] = X + m * K + 8 * c;
  }
  auto dma_x = [&](half8v* buf, int64_t h) {
    const int64_t koff = (h >> 1) * 256 + (h & 1) * 128;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) lds_load<16>(xsrc[i] + koff, buf + i * kThreads + wave * 64);
  };

  float4v acc[TA * B];
#pragma unroll
  for (int i = 0; i < TA * B; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};

  half8v afr[2][TA];
  half8v bfr[2][B];
  auto read_b = [&](half8v (&bf)[B], const half8v* buf, int jj) {
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const int mm = bi * 16 + r, c = 4 * jj + g;
      bf[bi] = buf[mm * 16 + (c ^ (mm & 15))];
    }
  };
  auto splice = [&](half8v (&dst)[TA], const WHalfL<F, TA>& wv, auto JC) {
    constexpr int jj = decltype(JC)::value;
#pragma unroll
    for (int a = 0; a < TA; ++a) dst[a] = Fmt<F>::template half_step<jj>(wv.h[a], s2[a]);
  };
  auto mfmas = [&](const half8v (&av)[TA], const half8v (&bf)[B]) {
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
        acc[a * B + bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bf[bi], acc[a * B + bi], 0, 0, 0);
  };
  auto interleave = [&](auto NDS) {  // as in tiled_run: next k-step's reads after 2 MFMAs
    constexpr int nds = decltype(NDS)::value;
#pragma unroll
    for (int i = 0; i < TA * B; ++i) {
      if constexpr (nds > 0) {
        if (i == 2) __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using IB = std::integral_constant<int, B>;
  auto vmcnt = [](auto NC) {
    constexpr int n = decltype(NC)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  };
  // Loads per step, in issue order: X(h+1) (kLoadsPerThread), then the
  // words of h+3 (kWLoads).  Before reading the words of h+1 at the end of
  // step h, the loads issued after them may still be in flight: X(h),
  // words(h+2), X(h+1), words(h+3).  Before the barrier: words(h+3).
  constexpr int kWLoads = TA * Fmt<F>::kStageLoads;
  using WaitW = std::integral_constant<int, 2 * kLoadsPerThread + 2 * kWLoads>;
  using WaitX = std::integral_constant<int, kWLoads>;

  // One half-tile h: k-steps 0..3 from X buffer `xc` and words `wc`; copy
  // X(h+1) into `xn` and the words of h+3 into stage `wt`; read the words of
  // h+1 from stage `wr` into `wn` and splice its first k-step while the
  // last k-step's MFMAs run.
  auto step = [&](const half8v* xc, half8v* xn, u32x4* wt, u32x4* wr, const WHalfL<F, TA>& wc,
                  WHalfL<F, TA>& wn, int64_t hx, int64_t hw) {
    dma_x(xn, hx);
    stage_w(wt, hw);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[0], xc, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[1], xc, 1); splice(afr[1], wc, I1{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[0], xc, 2); splice(afr[0], wc, I2{}); mfmas(afr[1], bfr[1]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);
    vmcnt(WaitW{});
    read_w(wn, wr);
    read_b(bfr[1], xc, 3); splice(afr[1], wc, I3{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);
                           splice(afr[0], wn, I0{}); mfmas(afr[1], bfr[1]); interleave(I0{});
    __builtin_amdgcn_sched_barrier(0);
    vmcnt(WaitX{});
    barrier_no_fence();
  };

  const int64_t h0 = 2 * kt0, h1 = 2 * kt1;  // half-tiles of this split
  if (h0 < h1) {
    // Prefetch indices are clamped to the split's last half-tile, so every
    // step issues the same loads (the wait counts are constants).  The loop
    // body is four steps (one turn of both rings); the remaining one to
    // three steps follow it.
    auto cl = [&](int64_t h) { return h < h1 - 1 ? h : h1 - 1; };
    // Issue order words(h0), words(h0+1), X(h0), words(h0+2): from the
    // first step on, the words of h+1 are followed by X(h), words(h+2),
    // X(h+1), words(h+3), as the wait counts assume.
    WHalfL<F, TA> wa, wb;
    stage_w(wl0, h0);
    stage_w(wl1, cl(h0 + 1));
    dma_x(xb0, h0);
    stage_w(wl2, cl(h0 + 2));
    vmcnt(WaitX{});  // X(h0) and the words of h0 (issued before it) have landed
    barrier_no_fence();
    read_w(wa, wl0);
    splice(afr[0], wa, I0{});
    int64_t h = h0;
    for (; h + 4 <= h1; h += 4) {
      step(xb0, xb1, wl3, wl1, wa, wb, cl(h + 1), cl(h + 3));
      step(xb1, xb0, wl0, wl2, wb, wa, cl(h + 2), cl(h + 4));
      step(xb0, xb1, wl1, wl3, wa, wb, cl(h + 3), cl(h + 5));
      step(xb1, xb0, wl2, wl0, wb, wa, cl(h + 4), cl(h + 6));
    }
    if (h < h1) step(xb0, xb1, wl3, wl1, wa, wb, cl(h + 1), cl(h + 3));
    if (h + 1 < h1) step(xb1, xb0, wl0, wl2, wb, wa, cl(h + 2), cl(h + 4));
    if (h + 2 < h1) step(xb0, xb1, wl1, wl3, wa, wb, cl(h + 3), cl(h + 5));
    // No copy into LDS may still be in flight when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(0);
  }

  if (splits > 1) {
    const int64_t unit = (mg * ntiles + nt) * NW + wave;
    float* unit_part = part + unit * static_cast<int64_t>(splits) * (TA * B * 256);
    if (!splitk_fixup<TA * B, true>(acc, unit_part, counters + unit, split, splits, lane)) return;
  }
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    const int64_t nb = nt * 16 + wave * TA + a;
    if (nb >= nblocks) continue;
#pragma unroll
    for (int bi = 0; bi < B; ++bi)
      store_y_block(Y, acc[a * B + bi], m0 + bi * 16 + r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel with whole-tile stages (16 < M <= 64): as fp6_gemm_tiled, but
// each pipeline stage is a whole 256-k tile (8 k-steps) instead of a half,
// so the X copy and the packed words of the next tile have twice the compute
// time to arrive, and there is one barrier per tile.  X stages are BM x 256
// (32 KB at BM = 64, two of them).  Measured on MI355X (OPT-30B QKV, M=64):
// 10% faster than half-tile stages; at BM = 128 (M >= 128) it is not.
// ---------------------------------------------------------------------------
template <int F, int TA>
struct WTile {
  typename Fmt<F>::Tile t[TA];
};

template <int F, int B, int TA, int NW>
__global__ __launch_bounds__(64 * NW) void fp6_gemm_tiledw(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  constexpr int BM = 16 * B;
  constexpr int kUnits = BM * 32;                 // 16-byte units per X stage (BM x 256)
  constexpr int kThreads = 64 * NW;
  static_assert(TA * NW == 16, "a workgroup covers 16 row blocks");
  constexpr int kLoadsPerThread = kUnits / kThreads;
  __shared__ __attribute__((aligned(16))) half8v xbuf0[kUnits];
  __shared__ __attribute__((aligned(16))) half8v xbuf1[kUnits];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 8;
  const int64_t kstr = nblocks * Fmt<F>::kTileQuads;  // quads between k-tiles of a row block
  const int64_t ntiles = (nblocks + 15) >> 4;     // 256-row workgroup tiles
  const uint32_t lb = static_cast<uint32_t>(xcd_logical_block(blockIdx.x, gridDim.x));
  const int split = static_cast<int>(umod32(lb, splits));
  const uint32_t bidx = udiv32(lb, splits);
  const uint32_t bq = udiv32(bidx, static_cast<uint32_t>(ntiles));
  const int64_t nt = bidx - bq * static_cast<uint32_t>(ntiles);
  const int64_t mg = bq + mg_base;
  const int64_t kt0 = udiv32(split * static_cast<uint32_t>(ktiles), splits);
  const int64_t kt1 = udiv32((split + 1) * static_cast<uint32_t>(ktiles), splits);
  const int r = lane & 15, g = lane >> 4;
  const int64_t m0 = mg * BM;

  const u32x4* w[TA];
  int64_t srow[TA];
  half2v s2[TA];
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    int64_t nb = nt * 16 + wave * TA + a;
    if (nb >= nblocks) nb = nblocks - 1;
    w[a] = wp + nb * Fmt<F>::kTileQuads + lane;
    srow[a] = nb * 16 + r;
  }
  auto load_wt = [&](WTile<F, TA>& st, int64_t kt) {
#pragma unroll
    for (int a = 0; a < TA; ++a) Fmt<F>::load(st.t[a], w[a] + kt * kstr, lane);
  };

  // X direct loads: instruction i of this wave fills LDS units
  // [i*kThreads + wave*64, +64) linearly; unit u = (row mm = u/32, slot
  // c' = u%32) receives global chunk c = c' ^ (mm & 15) of X row m0+mm.
  const _Float16* xsrc[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int u = i * kThreads + tid, mm = u >> 5, c = (u & 31) ^ (mm & 15);
    int64_t m = m0 + mm;
    if (m >= M) m = M - 1;
    xsrc[i] = X + m * K + 8 * c;
  }
  auto dma_x = [&](half8v* buf, int64_t kt) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(xsrc[i] + kt * 256),
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(buf + i * kThreads + wave * 64)),
          16, 0, 0);
  };

  float4v acc[TA * B];
#pragma unroll
  for (int i = 0; i < TA * B; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};

  half8v afr[2][TA];
  half8v bfr[2][B];
  auto read_b = [&](half8v (&bf)[B], const half8v* buf, int j) {
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const int mm = bi * 16 + r, c = 4 * j + g;
      bf[bi] = buf[mm * 32 + (c ^ (mm & 15))];
    }
  };
  auto splice = [&](half8v (&dst)[TA], const WTile<F, TA>& wt, auto JC) {
    constexpr int j = decltype(JC)::value;
#pragma unroll
    for (int a = 0; a < TA; ++a) dst[a] = Fmt<F>::template step<j>(wt.t[a], s2[a]);
  };
  auto mfmas = [&](const half8v (&av)[TA], const half8v (&bf)[B]) {
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
        acc[a * B + bi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bf[bi], acc[a * B + bi], 0, 0, 0);
  };
  // The next k-step's B reads go first here: with 64 columns (8 MFMAs per
  // k-step) the ordering of fp6_gemm_tiled measured 3% slower.
  auto interleave = [&](auto NDS) {
    constexpr int nds = decltype(NDS)::value;
    if constexpr (nds > 0) __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);
#pragma unroll
    for (int i = 0; i < TA * B; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using IB = std::integral_constant<int, B>;
  constexpr int kWLoads = TA * Fmt<F>::kTileLoads;
  constexpr int kWaitDma = (kWLoads & 15) | ((kWLoads >> 4) << 14) | (7 << 4) | (15 << 8);

  // One tile: k-steps 0..7 from buffer `cur`; prefetch X(kt+1) into `nxt`
  // and the words of kt+1 into `wn`; overlap the last k-step with the splice
  // of kt+1's first k-step.
  auto tile_step = [&](half8v* cur, half8v* nxt, const WTile<F, TA>& wc, WTile<F, TA>& wn, int64_t knext) {
    dma_x(nxt, knext);
    __builtin_amdgcn_sched_barrier(0);
    load_wt(wn, knext);
    __builtin_amdgcn_sched_barrier(0);
    read_b(bfr[0], cur, 0);
    read_b(bfr[1], cur, 1); splice(afr[1], wc, std::integral_constant<int, 1>{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    read_b(bfr[0], cur, 2); splice(afr[0], wc, std::integral_constant<int, 2>{}); mfmas(afr[1], bfr[1]); interleave(IB{});
    read_b(bfr[1], cur, 3); splice(afr[1], wc, std::integral_constant<int, 3>{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    read_b(bfr[0], cur, 4); splice(afr[0], wc, std::integral_constant<int, 4>{}); mfmas(afr[1], bfr[1]); interleave(IB{});
    read_b(bfr[1], cur, 5); splice(afr[1], wc, std::integral_constant<int, 5>{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    read_b(bfr[0], cur, 6); splice(afr[0], wc, std::integral_constant<int, 6>{}); mfmas(afr[1], bfr[1]); interleave(IB{});
    read_b(bfr[1], cur, 7); splice(afr[1], wc, std::integral_constant<int, 7>{}); mfmas(afr[0], bfr[0]); interleave(IB{});
    __builtin_amdgcn_sched_barrier(0);  // keep the splice of kt+1 last (see fp6_gemm_tiled)
                            splice(afr[0], wn, std::integral_constant<int, 0>{}); mfmas(afr[1], bfr[1]); interleave(I0{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitDma);
    __syncthreads();
  };

  if (kt0 < kt1) {
    auto clampk = [&](int64_t t) { return t < kt1 - 1 ? t : kt1 - 1; };
    WTile<F, TA> wa, wb;
    dma_x(xbuf0, kt0);
    load_wt(wa, kt0);
    __builtin_amdgcn_sched_barrier(0);  // first loads, then the row scales, one round trip
#pragma unroll
    for (int a = 0; a < TA; ++a) s2[a] = row_scale2<F>(scales, srow[a]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[0], wa, std::integral_constant<int, 0>{});
    int64_t kt = kt0;
    for (; kt + 2 <= kt1; kt += 2) {
      tile_step(xbuf0, xbuf1, wa, wb, clampk(kt + 1));
      tile_step(xbuf1, xbuf0, wb, wa, clampk(kt + 2));
    }
    if (kt < kt1) tile_step(xbuf0, xbuf1, wa, wb, clampk(kt + 1));
  }

  if (splits > 1) {
    const int64_t unit = (mg * ntiles + nt) * NW + wave;
    float* unit_part = part + unit * static_cast<int64_t>(splits) * (TA * B * 256);
    if (!splitk_fixup<TA * B, true>(acc, unit_part, counters + unit, split, splits, lane)) return;
  }
#pragma unroll
  for (int a = 0; a < TA; ++a) {
    const int64_t nb = nt * 16 + wave * TA + a;
    if (nb >= nblocks) continue;
#pragma unroll
    for (int bi = 0; bi < B; ++bi)
      store_y_block(Y, acc[a * B + bi], m0 + bi * 16 + r, M, N, nb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// Launchers (host code), one instantiation per format.
// ---------------------------------------------------------------------------
template <int F, int KTW, int WK>
int launch_ksplit_t(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                    int64_t K, int splits, float* part, unsigned* cnt, int cus, hipStream_t stream) {
  const int64_t nblocks = N >> 4;
  // Workgroups per split: one per CU in all, at most one per row block.
  int64_t per_split = cus / splits;
  if (per_split < 1) per_split = 1;
  if (per_split > nblocks) per_split = nblocks;
  const dim3 grid(static_cast<unsigned>(per_split * splits));
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits};
  const void* kern = M == 1 ? reinterpret_cast<const void*>(&fp6_gemm_ksplit<F, KTW, WK, true>)
                            : reinterpret_cast<const void*>(&fp6_gemm_ksplit<F, KTW, WK>);
  if constexpr (KTW == 1) {
    // 2..8 row blocks per workgroup: the straight-line form (P = 6 or 8
    // covers 5..8, the busiest workgroups setting the count).
    const int64_t per_wg = fpx_ceil_div(nblocks, per_split);
#define FP6_KS_P(PP)                                                                       \
  kern = M == 1 ? reinterpret_cast<const void*>(&fp6_gemm_ksplit<F, 1, WK, true, PP>)      \
                : reinterpret_cast<const void*>(&fp6_gemm_ksplit<F, 1, WK, false, PP>)
    if (per_wg == 2) FP6_KS_P(2);
    else if (per_wg == 3) FP6_KS_P(3);
    else if (per_wg == 4) FP6_KS_P(4);
    else if (per_wg == 5 || per_wg == 6) FP6_KS_P(6);
    else if (per_wg == 7 || per_wg == 8) FP6_KS_P(8);
#undef FP6_KS_P
  }
  return hipLaunchKernel(kern, grid, dim3(64 * WK), args, 0, stream) == hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

// WK waves per workgroup; each wave holds ceil(K/256 / WK) k-tiles.
template <int F, int WK>
int launch_ksplit(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                  int64_t K, int splits, float* part, unsigned* cnt, int cus, hipStream_t stream) {
  // Tiles per wave: the longest split's k-tiles over the waves.
  const int64_t split_tiles = fpx_ceil_div(K >> 8, splits);
  switch (fpx_ceil_div(split_tiles, WK)) {
    case 1: return launch_ksplit_t<F, 1, WK>(X, W, S, Y, M, N, K, splits, part, cnt, cus, stream);
    case 2: return launch_ksplit_t<F, 2, WK>(X, W, S, Y, M, N, K, splits, part, cnt, cus, stream);
    case 3: if constexpr (WK == 8) return launch_ksplit_t<F, 3, WK>(X, W, S, Y, M, N, K, splits, part, cnt, cus, stream);
            return FP6_E_VALUE;
    case 4: if constexpr (WK == 8) return launch_ksplit_t<F, 4, WK>(X, W, S, Y, M, N, K, splits, part, cnt, cus, stream);
            return FP6_E_VALUE;
    default: return FP6_E_VALUE;
  }
}

template <int F, int KTW, int WK>
int launch_kslice_t(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                    int64_t K, int cus, hipStream_t stream) {
  (void)cus;
  const dim3 grid(static_cast<unsigned>(N >> 4));  // one workgroup per row block
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  void* args[] = {&x, &w, &sc, &y, &M, &N, &K};
  const void* kern = reinterpret_cast<const void*>(&fp6_gemm_kslice<F, KTW, WK>);
  if constexpr (KTW == 1) {
    if (M == 1) kern = reinterpret_cast<const void*>(&fp6_gemm_kslice<F, 1, WK, true>);
  }
  return hipLaunchKernel(kern, grid, dim3(64 * WK), args, 0, stream) == hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

// 8 waves up to K = 2048, else 16 waves with up to 3 k-tiles each.
template <int F>
int launch_kslice(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                  int64_t K, int cus, hipStream_t stream) {
  const int64_t kt = K >> 8;
  if (kt <= 8) return launch_kslice_t<F, 1, 8>(X, W, S, Y, M, N, K, cus, stream);
  if (kt <= 16) return launch_kslice_t<F, 1, 16>(X, W, S, Y, M, N, K, cus, stream);
  if (kt <= 32) return launch_kslice_t<F, 2, 16>(X, W, S, Y, M, N, K, cus, stream);
  if (kt <= 48) return launch_kslice_t<F, 3, 16>(X, W, S, Y, M, N, K, cus, stream);
  return FP6_E_VALUE;
}

// K-ring kernel: P = (row block, K-split) units per CU (rounded up, at most
// 8), one workgroup per P row blocks and K-split; each wave holds
// ceil(K/256 / splits / 8) <= 4 k-tiles.  With one k-tile per wave two row
// blocks are in flight (16x28672x2048 11.6 -> 10.9 us, 16x8192x2048 5.8 ->
// 5.6); with 2-3 that was 3-13% slower (16x11008x4096 9.3 -> 10.1 us).
template <int F>
int launch_kring(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                 int64_t K, int splits, float* part, unsigned* cnt, int cus, hipStream_t stream) {
  const int64_t nblocks = N >> 4;
  int P = static_cast<int>(fpx_ceil_div(nblocks * splits, cus));
  if (P < 1) P = 1;
  if (P > 8 || M > 16 || splits < 1) return FP6_E_VALUE;
  const dim3 grid(static_cast<unsigned>(fpx_ceil_div(nblocks, P) * splits));
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &P, &splits};
  const void* kern = nullptr;
  const bool m1 = M == 1;
#define FP6_KR_CASE(T)                                                                       \
  case T:                                                                                    \
    kern = m1 ? reinterpret_cast<const void*>(&fp6_gemm_kring<F, T, true, (T == 1 ? 2 : 1)>)  \
              : reinterpret_cast<const void*>(&fp6_gemm_kring<F, T, false, (T == 1 ? 2 : 1)>); \
    break;
  switch (fpx_ceil_div(fpx_ceil_div(K >> 8, splits), 8)) {
    FP6_KR_CASE(1) FP6_KR_CASE(2) FP6_KR_CASE(3) FP6_KR_CASE(4)
    default: return FP6_E_VALUE;
  }
#undef FP6_KR_CASE
  return hipLaunchKernel(kern, grid, dim3(512), args, 0, stream) == hipSuccess ? FP6_OK : FP6_E_HIP;
}

template <int F, int A, int D, int NW, int MB = 1>
int launch_xlds(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                int64_t K, int splits, float* part, unsigned* cnt, hipStream_t stream) {
  const int64_t ngroups = fpx_ceil_div(N >> 4, A), gsets = fpx_ceil_div(ngroups, NW);
  const int64_t mgroups = fpx_ceil_div(M, 16 * MB);
  const int64_t per_mg = gsets * splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_xlds<F, A, D, NW, MB>), grid, dim3(64 * NW),
                        args, 0, stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

template <int F, int A, int MB, int D>
int launch_stream(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                  int64_t K, int splits, float* part, unsigned* cnt, hipStream_t stream) {
  const int64_t ngroups = fpx_ceil_div(N >> 4, A), gquads = fpx_ceil_div(ngroups, 4);
  const int64_t mgroups = fpx_ceil_div(M, 16 * MB);
  // Keep each launch below 2^24 workgroups.
  const int64_t per_mg = gquads * splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    // The launch's own status (not the thread's sticky last error).
    if (hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_stream<F, A, MB, D>), grid, dim3(256),
                        args, 0, stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

template <int F, int B, int TA, int NW>
int launch_tiledw(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                  int64_t K, int splits, float* part, unsigned* cnt, hipStream_t stream) {
  const int64_t ntiles = fpx_ceil_div(N >> 4, 16);
  const int64_t mgroups = fpx_ceil_div(M, 16 * B);
  const int64_t per_mg = ntiles * splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_tiledw<F, B, TA, NW>), grid, dim3(64 * NW),
                        args, 0, stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

// Stream-K tiled kernel: one launch, `workgroups` workgroups (splits field
// of the plan), all m-groups.
template <int F, int B, int TA, int NW>
int launch_tiled_sk(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                    int64_t K, int workgroups, float* part, unsigned* cnt, hipStream_t stream) {
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  int unused = 0;
  int64_t unused64 = 0;
  void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &unused, &unused64};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_tiled_sk<F, B, TA, NW>),
                         dim3(static_cast<unsigned>(workgroups)), dim3(64 * NW), args, 0, stream) == hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

template <int F, int B, int TA, int NW>
int launch_tiledl(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                  int64_t K, int splits, float* part, unsigned* cnt, hipStream_t stream) {
  const int64_t ntiles = fpx_ceil_div(N >> 4, 16);
  const int64_t mgroups = fpx_ceil_div(M, 16 * B);
  const int64_t per_mg = ntiles * splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_tiledl<F, B, TA, NW>), grid, dim3(64 * NW),
                        args, 0, stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

template <int F, int B, int TA, int NW>
int launch_tiled(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                 int64_t K, int splits, float* part, unsigned* cnt, hipStream_t stream) {
  const int64_t ntiles = fpx_ceil_div(N >> 4, 16);
  const int64_t mgroups = fpx_ceil_div(M, 16 * B);
  const int64_t per_mg = ntiles * splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(X);
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* y = static_cast<_Float16*>(Y);
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&fp6_gemm_tiled<F, B, TA, NW>), grid, dim3(64 * NW),
                        args, 0, stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}


// The planned launch of one format.
template <int F>
int launch_variant(const fpx::LaunchCtx& c) {
  const void *X = c.X, *W = c.W, *S = c.S;
  void* Y = c.Y;
  const int64_t M = c.M, N = c.N, K = c.K;
  const int sp = c.splits;
  float* pt = c.part;
  unsigned* ct = c.counters;
  hipStream_t s = c.stream;
  switch (c.variant) {
    case 1: return launch_stream<F, 1, 1, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 2: return launch_stream<F, 1, 4, 2>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 3: return launch_stream<F, 2, 1, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 4: return launch_stream<F, 4, 1, 2>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 5: return launch_tiled<F, 4, 4, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 6: return launch_tiled<F, 8, 4, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 7: return launch_stream<F, 1, 1, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 8: return launch_stream<F, 2, 1, 6>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 9: return launch_ksplit<F, 8>(X, W, S, Y, M, N, K, sp, pt, ct, c.cus, s);
    case 10: return launch_tiled<F, 8, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 11: return launch_tiled<F, 4, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 12: return launch_ksplit<F, 16>(X, W, S, Y, M, N, K, sp, pt, ct, c.cus, s);
    case 13: return launch_kslice<F>(X, W, S, Y, M, N, K, c.cus, s);
    case 14: return launch_xlds<F, 2, 4, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 15: return launch_xlds<F, 1, 4, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 16: return launch_xlds<F, 2, 4, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 17: return launch_tiledw<F, 4, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 18: return launch_xlds<F, 1, 4, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 19: return launch_xlds<F, 2, 2, 8, 2>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 20: return launch_xlds<F, 2, 2, 8, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 21: return launch_xlds<F, 1, 4, 8, 2>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 22: return launch_xlds<F, 1, 2, 8, 4>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 23: return launch_tiledl<F, 8, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 24: return launch_tiledl<F, 4, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 25: return launch_tiled_sk<F, 8, 2, 8>(X, W, S, Y, M, N, K, sp, pt, ct, s);
    case 26: return launch_kring<F>(X, W, S, Y, M, N, K, sp, pt, ct, c.cus, s);
    default: return FP6_E_VALUE;
  }
}

// De-quantisation export: one wave per tile, 4 waves per workgroup.
template <int F>
int launch_dequant(const void* packed_W, const void* scales, void* W16, int64_t N, int64_t K,
                   hipStream_t stream) {
  const int64_t tiles = (N >> 4) * (K >> 8);
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
  const u32x4* w = static_cast<const u32x4*>(packed_W);
  const _Float16* sc = static_cast<const _Float16*>(scales);
  _Float16* out = static_cast<_Float16*>(W16);
  void* args[] = {&w, &sc, &out, &N, &K};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fp6_dequant_kernel<F>), grid, dim3(256), args, 0,
                         stream) == hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

}  // namespace

// Instantiates the launch entry points of one format inside namespace fpx.
#define FPX_DEFINE_FORMAT(NAME, F)                                                          \
  namespace fpx {                                                                           \
  int launch_##NAME(const LaunchCtx& c) { return launch_variant<F>(c); }                   \
  int dequant_##NAME(const void* W, const void* S, void* W16, int64_t N, int64_t K,         \
                     hipStream_t s) {                                                       \
    return launch_dequant<F>(W, S, W16, N, K, s);                                           \
  }                                                                                         \
  }
