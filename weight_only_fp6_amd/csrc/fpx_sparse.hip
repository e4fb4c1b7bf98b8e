// Kernels of the 2:4-sparse FP6 (e3m2) weight-only linear layer on gfx950
// sparse matrix cores.
//
// Sparse-Marlin (first page, post on quantised-weight kernels, points on 2:4
// sparsity): quantised weights that are also 2:4 structured-sparse, on sparse
// matrix units, with values, metadata and scales laid out together.
//
// gfx950 design:
//  * v_smfmac_f32_16x16x64_f16 multiplies a 16x64 A operand of which 2 of
//    every 4 k are kept (8 fp16 per lane, plus 2-bit positions in an index
//    VGPR) by a dense 64x16 B operand (16 fp16 per lane: lane 16g+r holds
//    column r, k = 16g..16g+15).  Lane 16g+r's A element i is kept weight i%2
//    of the dense group at k-offset 32(g%2) + 16(i/4) + 8(g/2) + 4((i%4)/2),
//    its position taken from bits 16*abid + 2i of the index VGPR.
//  * A packed tile covers 16 rows x 512 dense k (4096 bytes): the kept codes
//    in the order of a dense FP6 tile (so the FP6 splice and row-scale fold are
//    reused unchanged) and one 16-byte quad of positions per lane, whose word
//    j/2 is the index operand of k-steps j (abid 0) and j+1 (abid 1).  A wave
//    reads a tile with four coalesced 16-byte loads per lane.
//  * 0.5 bytes per dense weight instead of 0.75, and one sparse MFMA per 64
//    dense k instead of two dense ones.
#include "fpx_device.h"

namespace {

typedef _Float16 half16v __attribute__((ext_vector_type(16)));

constexpr int kSpTileQuads = 256;  // 16-byte units per 16 x 512 tile

struct SpTile {
  TileFp6 w;   // kept codes, FP6 layout
  u32x4 idx;   // positions: word j/2 = k-steps j (bits 0..15) and j+1 (16..31)
};

template <bool NT = false>
__device__ __forceinline__ void sp_load(SpTile& t, const u32x4* p, int lane) {
  Fmt<kE3M2>::template load<NT>(t.w, p, lane);
  t.idx = ldw<NT>(p + 192);
}

template <int J>
__device__ __forceinline__ float4v sp_mac(const SpTile& t, half2v s2, const half16v& b, float4v acc) {
  const half8v a = Fmt<kE3M2>::template step<J>(t.w, s2);
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, b, acc, static_cast<int>(t.idx[J >> 1]), 0, J & 1);
}

// ---------------------------------------------------------------------------
// K-slice kernel (M <= 16, few row blocks): one workgroup per row block, its
// WK waves take one sparse tile each (K <= WK*512), reduce through LDS.
// ---------------------------------------------------------------------------
template <int WK>
__global__ __launch_bounds__(64 * WK) void sp_gemm_kslice(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, int64_t M, int64_t N,
    int64_t K) {
  __shared__ float4v red[WK][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 9;
  const int64_t nb = blockIdx.x;
  if (nb >= nblocks) return;  // uniform for the workgroup
  const int64_t kw0 = wave * ktiles / WK, kw1 = (wave + 1) * ktiles / WK;  // at most one tile
  const bool active = kw1 > kw0;
  const int64_t kt = active ? kw0 : 0;
  SpTile st;
  sp_load<true>(st, wp + (nb * ktiles + kt) * kSpTileQuads + lane, lane);
  // B operand rows m = r; rows >= M read row M-1 (their columns are never stored)
  const int64_t m = r < M ? r : M - 1;
  const _Float16* xrow = X + m * K + kt * 512 + 16 * g;
  half16v xf[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) xf[j] = *reinterpret_cast<const half16v*>(xrow + 64 * j);
  const half2v s2 = row_scale2<kE3M2>(scales, nb * 16 + r);
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    acc = sp_mac<0>(st, s2, xf[0], acc);
    acc = sp_mac<1>(st, s2, xf[1], acc);
    acc = sp_mac<2>(st, s2, xf[2], acc);
    acc = sp_mac<3>(st, s2, xf[3], acc);
    acc = sp_mac<4>(st, s2, xf[4], acc);
    acc = sp_mac<5>(st, s2, xf[5], acc);
    acc = sp_mac<6>(st, s2, xf[6], acc);
    acc = sp_mac<7>(st, s2, xf[7], acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) store_y_block(Y, reduce_waves<WK>(red, lane), r, M, N, nb * 16, g);
}

// ---------------------------------------------------------------------------
// K-split kernel (M <= 16, at most 8 row blocks per workgroup): the dense
// k-split kernel's straight-line form on sparse tiles.  A workgroup of 8
// waves takes K-split blockIdx % splits (at most 8 tiles of 512 k, one per
// wave) of the row blocks blockIdx / splits, + stride, ... (P of them at
// most).  Each wave stages its X slice (16 rows x 512 k = 16 KB) once,
// through its own LDS region with coalesced 1 KB row loads (32-byte units
// XOR-swizzled by row, so the 16 lanes of a B-fragment read hit distinct
// banks; at M = 1 one 16-byte load per lane and broadcast reads), keeps up
// to 4 row blocks' tiles in flight, multiplies every row block into a
// partial slot of its region, and after one barrier wave i sums row block i
// (through the fixed-order split-K fix-up when splits > 1).
// ---------------------------------------------------------------------------
template <int P, bool M1>
__global__ __launch_bounds__(512) void sp_gemm_ksplit(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits) {
  constexpr int WK = 8;
  static_assert(P >= 1 && P <= WK, "one summing wave per row block");
  __shared__ __attribute__((aligned(32))) half8v xw[WK][1024];  // 16 KB per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 9;
  const int split = static_cast<int>(blockIdx.x % splits);
  const int64_t kt0 = split * ktiles / splits, kts = (split + 1) * ktiles / splits - kt0;
  const int64_t kw0 = kt0 + wave * kts / WK, kw1 = kt0 + (wave + 1) * kts / WK;
  const bool active = kw1 > kw0;  // at most one tile per wave
  const int64_t kt = active ? kw0 : 0;
  const int64_t stride = gridDim.x / splits;
  const int64_t nb = blockIdx.x / splits;
  if (nb >= nblocks) return;  // uniform for the workgroup
  const int64_t nlast = nb + ((nblocks - 1 - nb) / stride) * stride;
  auto rb_of = [&](int i) {
    const int64_t nbi = nb + i * stride;
    return nbi < nlast ? nbi : nlast;
  };
  auto red_at = [&](int slot, int w) { return reinterpret_cast<float4v*>(&xw[w][64 * slot]); };

  // X loads first (the LDS writes below wait for them, not for the tiles).
  constexpr int kXLoads = M1 ? 1 : 16;
  half8v xg[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int64_t m = i < M ? i : M - 1;
    xg[i] = *reinterpret_cast<const half8v*>(X + m * K + kt * 512 + 8 * lane);
  }
  // Straight-line code throughout: a workgroup with fewer than P row
  // blocks repeats its last one, and an empty k-range is zeroed after its
  // products (behind a branch the compiler sinks loads past earlier waits).
  constexpr int S = P < 4 ? P : 4;
  SpTile ast[S];
  _Float16 asc[S];
  auto load_rb = [&](int st, int64_t rb) {
    sp_load<true>(ast[st], wp + (rb * ktiles + kt) * kSpTileQuads + lane, lane);
    asc[st] = scales[rb * 16 + r];
  };
#pragma unroll
  for (int i = 0; i < S; ++i) load_rb(i, rb_of(i));
  __builtin_amdgcn_sched_barrier(0);
  // Stage X: row rr's 32-byte unit u sits at unit u ^ rr of the row.
  half16v xf[8];
  if constexpr (M1) {
    xw[wave][lane] = xg[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = *reinterpret_cast<const half16v*>(&xw[wave][2 * (4 * j + g)]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) xw[wave][i * 64 + 2 * ((lane >> 1) ^ i) + (lane & 1)] = xg[i];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      xf[j] = *reinterpret_cast<const half16v*>(&xw[wave][r * 64 + 2 * ((4 * j + g) ^ r)]);
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const SpTile& st = ast[i % S];
    const half2v s2 = scale2_of<kE3M2>(asc[i % S]);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    acc = sp_mac<0>(st, s2, xf[0], acc);
    acc = sp_mac<1>(st, s2, xf[1], acc);
    acc = sp_mac<2>(st, s2, xf[2], acc);
    acc = sp_mac<3>(st, s2, xf[3], acc);
    acc = sp_mac<4>(st, s2, xf[4], acc);
    acc = sp_mac<5>(st, s2, xf[5], acc);
    acc = sp_mac<6>(st, s2, xf[6], acc);
    acc = sp_mac<7>(st, s2, xf[7], acc);
    if (!active) acc = float4v{0.f, 0.f, 0.f, 0.f};
    red_at(i, wave)[lane] = acc;
    if (i + S < P) load_rb(i % S, rb_of(i + S));
  }
  __syncthreads();
  if (wave < P && nb + wave * stride <= nlast) {  // repeated row blocks are not stored again
    const int64_t rb = nb + wave * stride;
    float4v sum = red_at(wave, 0)[lane];
#pragma unroll
    for (int w = 1; w < WK; ++w) sum += red_at(wave, w)[lane];
    if (splits > 1) {
      float4v a1[1] = {sum};
      if (!splitk_fixup<1>(a1, part + rb * splits * 256, counters + rb, split, splits, lane)) return;
      sum = a1[0];
    }
    store_y_block(Y, sum, r, M, N, rb * 16, g);
  }
}

// ---------------------------------------------------------------------------
// K-ring kernel on sparse tiles (M <= 16, K <= 8192, at most 8 row blocks
// per CU): the dense k-ring kernel's schedule.  One 8-wave workgroup per P
// consecutive row blocks over the whole K range; wave w owns the sparse
// tiles [w*KT/8, (w+1)*KT/8) (at most KTW) with their X fragments resident
// in registers (staged once through the wave's 16 KB LDS region; at M = 1
// the row is stored once and the fragments are broadcast reads), and walks
// the row blocks through a register ring of KTW tiles (R row blocks in
// flight), refilling slot t right after its products.  Partial tiles go to
// the wave's LDS region; after one barrier wave i sums row block i in wave
// order.  Tiles past a wave's range are stand-ins multiplied by zero X.
// ---------------------------------------------------------------------------
template <int KTW, bool M1, int R>
__global__ __launch_bounds__(512) void sp_gemm_kring(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int P) {
  constexpr int kWaves = 8;
  __shared__ __attribute__((aligned(32))) half8v xw[kWaves][1024];  // 16 KB per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t nblocks = N >> 4, ktiles = K >> 9;
  const int64_t kw0 = wave * ktiles / kWaves, kw1 = (wave + 1) * ktiles / kWaves;
  const int ktw = static_cast<int>(kw1 - kw0);  // 0..KTW sparse tiles for this wave
  const int64_t nb0 = static_cast<int64_t>(blockIdx.x) * P;
  if (nb0 >= nblocks) return;  // uniform for the workgroup
  const int pw = static_cast<int>(nblocks - nb0 < P ? nblocks - nb0 : P);
  const int64_t nb_last = nb0 + pw - 1;
  auto tile_of = [&](int t) -> int64_t {
    if (ktw == 0) return 0;
    return kw0 + (t < ktw ? t : ktw - 1);
  };
  // X of this wave's tiles first (row i of a tile: 16 bytes per lane).
  constexpr int kXLoads = M1 ? 1 : 16;
  half8v xg[KTW][kXLoads];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int64_t m = i < M ? i : M - 1;
      xg[t][i] = *reinterpret_cast<const half8v*>(X + m * K + tile_of(t) * 512 + 8 * lane);
    }
  }
  // The first R row blocks' tiles, each row scale after its first tile (the
  // loop's order, so the wait counts at its head are exact).
  SpTile ring[R][KTW];
  _Float16 sc[R];
  auto tile_ptr = [&](int64_t nb, int t) { return wp + (nb * ktiles + tile_of(t)) * kSpTileQuads + lane; };
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const int64_t nb = nb0 + rr < nb_last ? nb0 + rr : nb_last;
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      sp_load<true>(ring[rr][t], tile_ptr(nb, t), lane);
      if (t == 0) sc[rr] = scales[nb * 16 + r];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Stage X: row rr's 32-byte unit u sits at unit u ^ rr of the row.
  half16v xf[KTW][8];
#pragma unroll
  for (int t = 0; t < KTW; ++t) {
    const bool live = t < ktw;
    if constexpr (M1) {
      xw[wave][lane] = xg[t][0];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half16v v = *reinterpret_cast<const half16v*>(&xw[wave][2 * (4 * j + g)]);
        xf[t][j] = live ? v : half16v{};
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) xw[wave][i * 64 + 2 * ((lane >> 1) ^ i) + (lane & 1)] = xg[t][i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const half16v v = *reinterpret_cast<const half16v*>(&xw[wave][r * 64 + 2 * ((4 * j + g) ^ r)]);
        xf[t][j] = live ? v : half16v{};
      }
    }
  }
  auto row_block = [&](int i, auto SLOT, auto NEXT) {
    constexpr int kSlot = decltype(SLOT)::value;
    constexpr bool kNext = decltype(NEXT)::value;
    const half2v s2 = scale2_of<kE3M2>(sc[kSlot]);
    const int64_t nbn = nb0 + i + R < nb_last ? nb0 + i + R : nb_last;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KTW; ++t) {
      const SpTile& st = ring[kSlot][t];
      acc = sp_mac<0>(st, s2, xf[t][0], acc);
      acc = sp_mac<1>(st, s2, xf[t][1], acc);
      acc = sp_mac<2>(st, s2, xf[t][2], acc);
      acc = sp_mac<3>(st, s2, xf[t][3], acc);
      acc = sp_mac<4>(st, s2, xf[t][4], acc);
      acc = sp_mac<5>(st, s2, xf[t][5], acc);
      acc = sp_mac<6>(st, s2, xf[t][6], acc);
      acc = sp_mac<7>(st, s2, xf[t][7], acc);
      if constexpr (kNext) {
        // Fences keep the refill right after the tile's products.
        __builtin_amdgcn_sched_barrier(0);
        sp_load<true>(ring[kSlot][t], tile_ptr(nbn, t), lane);
        if (t == 0) sc[kSlot] = scales[nbn * 16 + r];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    reinterpret_cast<float4v*>(&xw[wave][64 * i])[lane] = acc;
  };
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
    float4v sum = reinterpret_cast<const float4v*>(&xw[0][64 * wave])[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += reinterpret_cast<const float4v*>(&xw[w][64 * wave])[lane];
    store_y_block(Y, sum, r, M, N, (nb0 + wave) * 16, g);
  }
}

// ---------------------------------------------------------------------------
// Streaming kernel with X shared through LDS (any M, in m-groups of 16).  A
// wave streams A row blocks over a K range through a register ring of D
// tiles; the NW waves of a workgroup share each X tile (16 rows x 512 k,
// 16 KB) through a 3-slot LDS ring, rows XOR-swizzled in 16-byte units; one
// barrier per tile.  Split-K fix-up as for the dense kernels.
// ---------------------------------------------------------------------------
template <int A, int D, int NW, int MB = 1>
__global__ __launch_bounds__(64 * NW) void sp_gemm_xlds(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  constexpr int kThreads = 64 * NW;
  constexpr int kChunks = MB * 16 * 64;  // 16-byte units per X tile (MB*16 rows x 512 k)
  constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) half8v xs[3][kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 9;
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
    w[a] = wp + (nb * ktiles) * kSpTileQuads + lane;
    s2[a] = row_scale2<kE3M2>(scales, nb * 16 + r);
  }
  // X staging: unit q = (row rr = q/64, chunk c = q%64) of the tile; rows
  // beyond M repeat row M-1 (their accumulator columns are never stored).
  const _Float16* xsrc[kPerThread];
  int xdst[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    int q = i * kThreads + tid;
    if (q >= kChunks) q = kChunks - 1;  // surplus threads duplicate the last unit
    const int rr = q >> 6, c = q & 63;
    int64_t m = mg * 16 * MB + rr;
    if (m >= M) m = M - 1;
    xsrc[i] = X + m * K + 8 * c;
    xdst[i] = rr * 64 + (c ^ (rr & 15));
  }
  half8v xstage[kPerThread];
  const int64_t klast = kt1 > kt0 ? kt1 - 1 : kt0;
  auto clampk = [&](int64_t t) { return t < klast ? t : klast; };
  auto gload_x = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      xstage[i] = *reinterpret_cast<const half8v*>(xsrc[i] + kt * 512);
  };
  auto swrite_x = [&](int slot) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) xs[slot][xdst[i]] = xstage[i];
  };

  float4v acc[A * MB];  // row block a, column group b: acc[a * MB + b]
#pragma unroll
  for (int i = 0; i < A * MB; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
  struct Stage {
    SpTile t[A];
  };
  auto load_w = [&](Stage& st, int64_t kt) {
#pragma unroll
    for (int a = 0; a < A; ++a) sp_load<MB == 1>(st.t[a], w[a] + kt * kSpTileQuads, lane);
  };
  auto mac = [&](const Stage& st, int slot) {
    const half8v* xb = xs[slot];
    // One column group: one B fragment per k-step (the form measured for
    // the M <= 16 default); several: each spliced k-step feeds MB MFMAs.
    if constexpr (MB == 1) {
#define FP6S_XL_STEP(J)                                                                  \
  {                                                                                      \
    const int c0 = (8 * J + 2 * g) ^ r;                                                  \
    const half8v lo = xb[r * 64 + c0], hi = xb[r * 64 + (c0 ^ 1)];                       \
    const half16v bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, \
                                               11, 12, 13, 14, 15);                      \
    _Pragma("unroll") for (int a = 0; a < A; ++a) acc[a] = sp_mac<J>(st.t[a], s2[a], bf, acc[a]); \
  }
      FP6S_XL_STEP(0) FP6S_XL_STEP(1) FP6S_XL_STEP(2) FP6S_XL_STEP(3)
      FP6S_XL_STEP(4) FP6S_XL_STEP(5) FP6S_XL_STEP(6) FP6S_XL_STEP(7)
    } else {
#define FP6S_XL_STEPM(J)                                                                  \
  {                                                                                      \
    const int c0 = (8 * J + 2 * g) ^ r;                                                  \
    half16v bf[MB];                                                                      \
    _Pragma("unroll") for (int b = 0; b < MB; ++b) {                                     \
      const half8v lo = xb[(b * 16 + r) * 64 + c0], hi = xb[(b * 16 + r) * 64 + (c0 ^ 1)]; \
      bf[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, \
                                      14, 15);                                           \
    }                                                                                    \
    _Pragma("unroll") for (int a = 0; a < A; ++a) {                                      \
      const half8v wa = Fmt<kE3M2>::template step<J>(st.t[a].w, s2[a]);                  \
      _Pragma("unroll") for (int b = 0; b < MB; ++b) acc[a * MB + b] =                   \
          __builtin_amdgcn_smfmac_f32_16x16x64_f16(wa, bf[b], acc[a * MB + b],           \
                                                   static_cast<int>(st.t[a].idx[J >> 1]), 0, J & 1); \
    }                                                                                    \
  }
      FP6S_XL_STEPM(0) FP6S_XL_STEPM(1) FP6S_XL_STEPM(2) FP6S_XL_STEPM(3)
      FP6S_XL_STEPM(4) FP6S_XL_STEPM(5) FP6S_XL_STEPM(6) FP6S_XL_STEPM(7)
    }
#undef FP6S_XL_STEPM
#undef FP6S_XL_STEP
  };

  // Tile i of the split uses slot i % 3.  Iteration i writes X(i+1) (loaded
  // during iteration i-1) into slot (i+1) % 3, whose last reader was
  // iteration i-2, loads X(i+2), consumes the ring stage of tile i and
  // refills it, then meets the barrier.  X stays one tile ahead here (unlike
  // the dense kernel): X at the ring's distance needs more registers than
  // two waves per SIMD allow with 16 KB sparse X tiles, and measured slower.
  // Branch-free steady state with clamped prefetch indices, the last (< D)
  // tiles in a tail.
  Stage ring[D];
  if (kt0 < kt1) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_w(ring[d], clampk(kt0 + d));
    gload_x(kt0);
    swrite_x(0);
    gload_x(clampk(kt0 + 1));
    __syncthreads();
    int64_t kt = kt0;
    int slot = 0;
    for (; kt + D <= kt1; kt += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int64_t t = kt + d;
        const int nslot = slot == 2 ? 0 : slot + 1;
        swrite_x(nslot);
        gload_x(clampk(t + 2));
        mac(ring[d], slot);
        load_w(ring[d], clampk(t + D));
        __syncthreads();
        slot = nslot;
      }
    }
#pragma unroll
    for (int d = 0; d + 1 < D; ++d) {
      if (kt + d < kt1) {
        const int nslot = slot == 2 ? 0 : slot + 1;
        swrite_x(nslot);
        gload_x(clampk(kt + d + 2));
        mac(ring[d], slot);
        __syncthreads();
        slot = nslot;
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
// Tiled kernel (M > 16): the dense tiled kernel's schedule on sparse tiles.
// Workgroup = NW waves x TA row blocks = 256 weight rows, BM = 16*B columns
// of X.  Per half-tile (4 sparse k-steps = 256 dense k): X (BM x 256) is
// copied global -> LDS with direct LDS loads, XOR-swizzled in 16-byte units;
// the packed words of the next half-tile (codes and positions) are loaded
// into registers; each k-step's A fragments are spliced once and reused for
// B sparse MFMAs while the next k-step is spliced.
// ---------------------------------------------------------------------------
struct SpHalf {
  u32x2 q2;   // 2-bit code words of k-steps 4h'..4h'+3
  u32x4 q4;   // 4-bit code words, one per k-step
  u32x2 idx;  // position words: k-steps (4h', 4h'+1) and (4h'+2, 4h'+3)
};

template <int TA>
struct SpWHalf {
  SpHalf h[TA];
};

template <int B, int TA, int NW>
__global__ __launch_bounds__(64 * NW) void sp_gemm_tiled(
    const _Float16* __restrict__ X, const u32x4* __restrict__ wp,
    const _Float16* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int64_t M, int64_t N, int64_t K, int splits,
    int64_t mg_base) {
  constexpr int BM = 16 * B;
  constexpr int kHalfUnits = BM * 32;             // 16-byte units per X half-tile buffer
  constexpr int kThreads = 64 * NW;
  static_assert(TA * NW == 16, "a workgroup covers 16 row blocks");
  constexpr int kLoadsPerThread = kHalfUnits / kThreads;
  __shared__ __attribute__((aligned(16))) half8v xbuf0[kHalfUnits];
  __shared__ __attribute__((aligned(16))) half8v xbuf1[kHalfUnits];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblocks = N >> 4, ktiles = K >> 9;
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
    w[a] = wp + (nb * ktiles) * kSpTileQuads + lane;
    srow[a] = nb * 16 + r;
  }
  auto load_wh = [&](SpWHalf<TA>& st, int64_t h) {  // half-tile h: tile h>>1, half h&1
    const int64_t kt = h >> 1;
    const int hh = static_cast<int>(h & 1);
#pragma unroll
    for (int a = 0; a < TA; ++a) {
      const u32x4* p = w[a] + kt * kSpTileQuads;
      st.h[a].q2 = reinterpret_cast<const u32x2*>(p)[hh];
      st.h[a].q4 = p[64 + 64 * hh];
      st.h[a].idx = reinterpret_cast<const u32x2*>(p + 192)[hh];
    }
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
  auto dma_x = [&](half8v* buf, int64_t h) {
    const int64_t koff = (h >> 1) * 512 + (h & 1) * 256;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i)
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(xsrc[i] + koff),
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(buf + i * kThreads + wave * 64)),
          16, 0, 0);
  };

  float4v acc[TA * B];
#pragma unroll
  for (int i = 0; i < TA * B; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};

  half8v afr[2][TA];
  half16v bfr[B];
  auto read_b1 = [&](const half8v* buf, int jj, int bi) {
    const int mm = bi * 16 + r;
    const int s0 = (8 * jj + 2 * g) ^ (mm & 15);
    bfr[bi] = __builtin_shufflevector(buf[mm * 32 + s0], buf[mm * 32 + (s0 ^ 1)], 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                      9, 10, 11, 12, 13, 14, 15);
  };
  auto read_b = [&](const half8v* buf, int jj) {
#pragma unroll
    for (int bi = 0; bi < B; ++bi) read_b1(buf, jj, bi);
  };
  auto splice = [&](half8v (&dst)[TA], const SpWHalf<TA>& wh, auto JC) {
    constexpr int jj = decltype(JC)::value;
#pragma unroll
    for (int a = 0; a < TA; ++a) dst[a] = splice6<kE3M2, jj & 1>(wh.h[a].q2[jj >> 1], wh.h[a].q4[jj], s2[a]);
  };
  // One k-step's products.  With RD, column group bi's fragment of k-step jn
  // is read into bfr[bi] right after the last product that uses it, so the
  // next k-step's reads overlap this one's products in the same registers
  // (two fragment sets would not fit).  Schedule: 1 MFMA then 3 VALU (the
  // next splice); with RD the last row block's MFMAs take the 2 LDS reads
  // of one fragment and 2 VALU each.
  auto mfmas = [&](const half8v (&av)[TA], const SpWHalf<TA>& wh, auto JC, const half8v* buf, int jn,
                   auto RD) {
    constexpr int jj = decltype(JC)::value;
    constexpr bool rd = decltype(RD)::value;
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int bi = 0; bi < B; ++bi) {
        acc[a * B + bi] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(
            av[a], bfr[bi], acc[a * B + bi], static_cast<int>(wh.h[a].idx[jj >> 1]), 0, jj & 1);
        if constexpr (rd) {
          if (a == TA - 1) read_b1(buf, jn, bi);
        }
      }
#pragma unroll
    for (int i = 0; i < (TA - 1) * B; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (rd) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, rd ? 2 : 3, 0);
    }
  };
  using RD1 = std::integral_constant<bool, true>;
  using RD0 = std::integral_constant<bool, false>;
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  // Wait for this wave's direct LDS loads of the next half-tile (issued
  // before the 3*TA weight loads of that half-tile), then the barrier makes
  // every wave's copy visible.
  constexpr int kWLoads = TA * 3;
  constexpr int kWaitDma = (kWLoads & 15) | ((kWLoads >> 4) << 14) | (7 << 4) | (15 << 8);

  // One half-tile: k-steps 0..3 from buffer `cur`; prefetch X(h+1) into
  // `nxt` and the words of h+1 into `wn`; the splice of the next k-step
  // (the last one: of h+1's first) overlaps the current k-step's MFMAs.
  auto half_step = [&](half8v* cur, half8v* nxt, const SpWHalf<TA>& wc, SpWHalf<TA>& wn, int64_t hnext) {
    dma_x(nxt, hnext);
    __builtin_amdgcn_sched_barrier(0);
    load_wh(wn, hnext);
    __builtin_amdgcn_sched_barrier(0);
    read_b(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[1], wc, J1{}); mfmas(afr[0], wc, J0{}, cur, 1, RD1{});
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[0], wc, J2{}); mfmas(afr[1], wc, J1{}, cur, 2, RD1{});
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[1], wc, J3{}); mfmas(afr[0], wc, J2{}, cur, 3, RD1{});
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[0], wn, J0{}); mfmas(afr[1], wc, J3{}, cur, 0, RD0{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitDma);
    __syncthreads();
  };

  const int64_t h0 = 2 * kt0, h1 = 2 * kt1;  // half-tiles of this split
  if (h0 < h1) {
    auto clamph = [&](int64_t h) { return h < h1 - 1 ? h : h1 - 1; };
    SpWHalf<TA> wa, wb;
    dma_x(xbuf0, h0);
    load_wh(wa, h0);
    __builtin_amdgcn_sched_barrier(0);  // first loads, then the row scales, one round trip
#pragma unroll
    for (int a = 0; a < TA; ++a) s2[a] = row_scale2<kE3M2>(scales, srow[a]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    splice(afr[0], wa, J0{});
    for (int64_t h = h0; h < h1; h += 2) {
      half_step(xbuf0, xbuf1, wa, wb, clamph(h + 1));
      half_step(xbuf1, xbuf0, wb, wa, clamph(h + 2));
    }
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
// De-quantisation export: one wave per tile; lane 16g+r writes, for each
// k-step, its 4 dense groups of row r (kept values at their positions, zeros
// elsewhere), so the 64 lanes cover the tile's 16 x 512 dense weights.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sp_dequant_kernel(const u32x4* __restrict__ wp,
                                                         const _Float16* __restrict__ scales,
                                                         _Float16* __restrict__ w16, int64_t N,
                                                         int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t ktiles = K >> 9;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (tile >= (N >> 4) * ktiles) return;
  const int64_t nb = tile / ktiles, kt = tile % ktiles;
  const int r = lane & 15, g = lane >> 4;
  SpTile st;
  sp_load(st, wp + tile * kSpTileQuads + lane, lane);
  const int64_t n = nb * 16 + r;
  const half2v s2 = row_scale2<kE3M2>(scales, n);
  _Float16* row = w16 + n * K + kt * 512;
  auto put = [&](auto JC, const half8v& a) {
    constexpr int j = decltype(JC)::value;
    const uint32_t iw = st.idx[j >> 1] >> (16 * (j & 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // the lane's groups: elements 2q, 2q+1
      const int off = 64 * j + 32 * (g & 1) + 16 * (q >> 1) + 8 * (g >> 1) + 4 * (q & 1);
      const int p0 = (iw >> (4 * q)) & 3, p1 = (iw >> (4 * q + 2)) & 3;
      half4v h;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h[e] = p0 == e ? a[2 * q] : (p1 == e ? a[2 * q + 1] : static_cast<_Float16>(0.0f));
      *reinterpret_cast<half4v*>(row + off) = h;
    }
  };
  put(std::integral_constant<int, 0>{}, Fmt<kE3M2>::template step<0>(st.w, s2));
  put(std::integral_constant<int, 1>{}, Fmt<kE3M2>::template step<1>(st.w, s2));
  put(std::integral_constant<int, 2>{}, Fmt<kE3M2>::template step<2>(st.w, s2));
  put(std::integral_constant<int, 3>{}, Fmt<kE3M2>::template step<3>(st.w, s2));
  put(std::integral_constant<int, 4>{}, Fmt<kE3M2>::template step<4>(st.w, s2));
  put(std::integral_constant<int, 5>{}, Fmt<kE3M2>::template step<5>(st.w, s2));
  put(std::integral_constant<int, 6>{}, Fmt<kE3M2>::template step<6>(st.w, s2));
  put(std::integral_constant<int, 7>{}, Fmt<kE3M2>::template step<7>(st.w, s2));
}

template <int WK>
int launch_sp_kslice(const fpx::LaunchCtx& c) {
  const dim3 grid(static_cast<unsigned>(c.N >> 4));  // one workgroup per row block
  const _Float16* x = static_cast<const _Float16*>(c.X);
  const u32x4* w = static_cast<const u32x4*>(c.W);
  const _Float16* sc = static_cast<const _Float16*>(c.S);
  _Float16* y = static_cast<_Float16*>(c.Y);
  int64_t M = c.M, N = c.N, K = c.K;
  void* args[] = {&x, &w, &sc, &y, &M, &N, &K};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sp_gemm_kslice<WK>), grid, dim3(64 * WK), args,
                         0, c.stream) == hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

// Workgroups per K-split and row blocks per workgroup of the sparse k-split
// kernel (one workgroup per CU in all).
int64_t sp_ksplit_per_split(int64_t N, int cus, int splits) {
  int64_t per_split = cus / splits;
  if (per_split < 1) per_split = 1;
  if (per_split > (N >> 4)) per_split = N >> 4;
  return per_split;
}

int launch_sp_ksplit(const fpx::LaunchCtx& c) {
  const int64_t per_split = sp_ksplit_per_split(c.N, c.cus, c.splits);
  const int64_t per_wg = fpx_ceil_div(c.N >> 4, per_split);
  const dim3 grid(static_cast<unsigned>(per_split * c.splits));
  const _Float16* x = static_cast<const _Float16*>(c.X);
  const u32x4* w = static_cast<const u32x4*>(c.W);
  const _Float16* sc = static_cast<const _Float16*>(c.S);
  _Float16* y = static_cast<_Float16*>(c.Y);
  float* part = c.part;
  unsigned* cnt = c.counters;
  int64_t M = c.M, N = c.N, K = c.K;
  int splits = c.splits;
  const void* kern = nullptr;
#define FP6_SPKS_P(PP)                                                                        \
  kern = M == 1 ? reinterpret_cast<const void*>(&sp_gemm_ksplit<PP, true>)                    \
                : reinterpret_cast<const void*>(&sp_gemm_ksplit<PP, false>)
  switch (per_wg) {
    case 1: FP6_SPKS_P(1); break;
    case 2: FP6_SPKS_P(2); break;
    case 3: FP6_SPKS_P(3); break;
    case 4: FP6_SPKS_P(4); break;
    case 5: case 6: FP6_SPKS_P(6); break;
    case 7: case 8: FP6_SPKS_P(8); break;
    default: return FP6_E_VALUE;
  }
#undef FP6_SPKS_P
  void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits};
  return hipLaunchKernel(kern, grid, dim3(512), args, 0, c.stream) == hipSuccess ? FP6_OK : FP6_E_HIP;
}

// Sparse k-ring: P = row blocks per CU (rounded up, <= 8); one sparse tile
// per wave up to K = 4096 (two row blocks in flight), two up to 8192.
int launch_sp_kring(const fpx::LaunchCtx& c) {
  const int64_t nblocks = c.N >> 4;
  int P = static_cast<int>(fpx_ceil_div(nblocks, c.cus));
  if (P < 1) P = 1;
  if (P > 8 || c.M > 16) return FP6_E_VALUE;
  const dim3 grid(static_cast<unsigned>(fpx_ceil_div(nblocks, P)));
  const _Float16* x = static_cast<const _Float16*>(c.X);
  const u32x4* w = static_cast<const u32x4*>(c.W);
  const _Float16* sc = static_cast<const _Float16*>(c.S);
  _Float16* y = static_cast<_Float16*>(c.Y);
  int64_t M = c.M, N = c.N, K = c.K;
  const bool m1 = M == 1;
  const void* kern = nullptr;
  switch (fpx_ceil_div(K >> 9, 8)) {
    case 1: kern = m1 ? reinterpret_cast<const void*>(&sp_gemm_kring<1, true, 2>)
                      : reinterpret_cast<const void*>(&sp_gemm_kring<1, false, 2>); break;
    case 2: kern = m1 ? reinterpret_cast<const void*>(&sp_gemm_kring<2, true, 1>)
                      : reinterpret_cast<const void*>(&sp_gemm_kring<2, false, 1>); break;
    default: return FP6_E_VALUE;
  }
  void* args[] = {&x, &w, &sc, &y, &M, &N, &K, &P};
  return hipLaunchKernel(kern, grid, dim3(512), args, 0, c.stream) == hipSuccess ? FP6_OK : FP6_E_HIP;
}

template <int A, int D, int NW, int MB = 1>
int launch_sp_xlds(const fpx::LaunchCtx& c) {
  const int64_t ngroups = fpx_ceil_div(c.N >> 4, A), gsets = fpx_ceil_div(ngroups, NW);
  const int64_t mgroups = fpx_ceil_div(c.M, 16 * MB);
  const int64_t per_mg = gsets * c.splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(c.X);
  const u32x4* w = static_cast<const u32x4*>(c.W);
  const _Float16* sc = static_cast<const _Float16*>(c.S);
  _Float16* y = static_cast<_Float16*>(c.Y);
  float* part = c.part;
  unsigned* cnt = c.counters;
  int64_t M = c.M, N = c.N, K = c.K;
  int splits = c.splits;
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&sp_gemm_xlds<A, D, NW, MB>), grid, dim3(64 * NW),
                        args, 0, c.stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

template <int B, int TA, int NW>
int launch_sp_tiled(const fpx::LaunchCtx& c) {
  const int64_t ntiles = fpx_ceil_div(c.N >> 4, 16);
  const int64_t mgroups = fpx_ceil_div(c.M, 16 * B);
  const int64_t per_mg = ntiles * c.splits;
  int64_t mg_chunk = ((int64_t(1) << 24) - 1) / per_mg;
  if (mg_chunk < 1) mg_chunk = 1;
  const _Float16* x = static_cast<const _Float16*>(c.X);
  const u32x4* w = static_cast<const u32x4*>(c.W);
  const _Float16* sc = static_cast<const _Float16*>(c.S);
  _Float16* y = static_cast<_Float16*>(c.Y);
  float* part = c.part;
  unsigned* cnt = c.counters;
  int64_t M = c.M, N = c.N, K = c.K;
  int splits = c.splits;
  for (int64_t mg0 = 0; mg0 < mgroups; mg0 += mg_chunk) {
    const int64_t nmg = (mgroups - mg0 < mg_chunk) ? (mgroups - mg0) : mg_chunk;
    const dim3 grid(static_cast<unsigned>(nmg * per_mg));
    int64_t mg_base = mg0;
    void* args[] = {&x, &w, &sc, &y, &part, &cnt, &M, &N, &K, &splits, &mg_base};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&sp_gemm_tiled<B, TA, NW>), grid, dim3(64 * NW),
                        args, 0, c.stream) != hipSuccess)
      return FP6_E_HIP;
  }
  return FP6_OK;
}

}  // namespace

namespace fpx {

int64_t sp_ksplit_rows_per_wg(int64_t N, int cus, int splits) {
  return fpx_ceil_div(N >> 4, sp_ksplit_per_split(N, cus, splits));
}

int launch_sparse(const LaunchCtx& c) {
  switch (c.variant) {
    case kSpKslice: return (c.K >> 9) <= 8 ? launch_sp_kslice<8>(c) : launch_sp_kslice<16>(c);
    case kSpXlds1: return launch_sp_xlds<1, 4, 4>(c);
    case kSpXlds2: return launch_sp_xlds<2, 4, 4>(c);
    case kSpTiled4: return launch_sp_tiled<4, 2, 8>(c);
    case kSpTiled8: return launch_sp_tiled<8, 2, 8>(c);
    case kSpKsplit: return launch_sp_ksplit(c);
    case kSpXldsMB1: return launch_sp_xlds<1, 4, 8, 2>(c);
    case kSpXldsMB2: return launch_sp_xlds<2, 2, 8, 2>(c);
    case kSpKring: return launch_sp_kring(c);
    default: return FP6_E_VALUE;
  }
}

int dequant_sparse(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s) {
  const int64_t tiles = (N >> 4) * (K >> 9);
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4));
  const u32x4* w = static_cast<const u32x4*>(W);
  const _Float16* sc = static_cast<const _Float16*>(S);
  _Float16* out = static_cast<_Float16*>(W16);
  void* args[] = {&w, &sc, &out, &N, &K};
  return hipLaunchKernel(reinterpret_cast<const void*>(&sp_dequant_kernel), grid, dim3(256), args, 0, s) ==
                 hipSuccess
             ? FP6_OK
             : FP6_E_HIP;
}

}  // namespace fpx
