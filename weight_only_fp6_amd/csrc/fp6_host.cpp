// Host side of the FPx weight-only linear layer: status strings, size rules,
// the row quantiser and the offline packer (layout v3) of every format.
//
// Plain C++17, no HIP calls: everything here runs on the CPU.
//
// TC-FPx explainer (duicuo.cn), section "redesigning the kernel solution":
// weights are re-ordered before inference and packed into aligned words, and
// each 6-bit weight is split into power-of-two pieces (2 + 4 bits) so the GPU
// can rebuild it with a few bit operations.  The concrete bit positions below
// are this library's own design for 64-lane wavefronts (see fp6.h).

#include "fp6.h"
#include "fp6s.h"
#include "fpx.h"
#include "fp6_limits.h"

#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// fp16 bit pattern -> double (exact).
double half_bits_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int exp = (h >> 10) & 0x1F;
  const int man = h & 0x3FF;
  double v;
  if (exp == 0) {
    v = std::ldexp(static_cast<double>(man), -24);
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(man + 1024), exp - 25);
  }
  return sign ? -v : v;
}

// double -> fp16 bits, one IEEE round-to-nearest-even.  Scaling by powers of
// two is exact, so nearbyint() (default rounding mode: ties to even) on the
// scaled value is the single rounding.
uint16_t double_to_half_rne(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // 65520 is the tie 65504|65536 -> even = inf
  if (a < 0x1p-14) {                        // subnormal binade (or zero)
    const double m = std::nearbyint(a * 0x1p24);
    return sign | static_cast<uint16_t>(m);  // m == 1024 is the smallest normal
  }
  int e;
  const double f = std::frexp(a, &e);       // a = f * 2^e, f in [0.5, 1)
  double r = std::nearbyint(f * 2048.0);    // 11-bit significand
  if (r == 2048.0) { r = 1024.0; ++e; }
  const int field = e + 14;
  if (field >= 31) return sign | 0x7C00;
  return sign | static_cast<uint16_t>((field << 10) | (static_cast<int>(r) - 1024));
}

// Weight formats: code width, mantissa bits, exponent bias, largest
// magnitude, and the bound on |scale| (the kernels fold s * 2^12 or s * 2^14
// into one fp16, exact only below it; FP4 multiplies by s itself).
struct FormatInfo {
  int bits, mbits, bias;
  double vmax, scale_limit;
};
constexpr double kInf = std::numeric_limits<double>::infinity();
constexpr FormatInfo kFormats[] = {
    {6, 2, 3, 28.0, 16.0},  // FPX_E3M2
    {6, 3, 1, 7.5, 4.0},    // FPX_E2M3
    {5, 2, 1, 7.0, 4.0},    // FPX_E2M2
    {4, 1, 1, 6.0, kInf},   // FPX_E2M1
};
constexpr int kNumFormats = sizeof(kFormats) / sizeof(kFormats[0]);

const FormatInfo* format_info(int format) {
  return format >= 0 && format < kNumFormats ? &kFormats[format] : nullptr;
}

// Nearest magnitude index of q >= 0 (index = e * 2^M + m), ties to the even
// index, saturating at the largest magnitude.  Values: m * 2^(1-bias-M) for
// e == 0 (subnormal), 2^(e-bias) * (1 + m / 2^M) for e >= 1.
int magnitude_index(const FormatInfo& f, double q) {
  const int nmag = 1 << (f.bits - 1);
  if (!(q < f.vmax)) return nmag - 1;        // also +inf
  if (q < std::ldexp(1.0, 1 - f.bias)) {     // subnormal grid
    // the first normal comes out as index 2^M, its own code
    return static_cast<int>(std::nearbyint(std::ldexp(q, f.bias - 1 + f.mbits)));
  }
  int E;
  const double fr = std::frexp(q, &E);       // q = fr * 2^E, fr in [0.5, 1)
  const double top = std::ldexp(1.0, f.mbits + 1);
  double r = std::nearbyint(fr * top);       // M+1 significant bits
  if (r == top) { r = top / 2; ++E; }
  // value = r / 2^(M+1) * 2^E = (2^M + m) / 2^M * 2^(E-1)  =>  e = E - 1 + bias
  const int idx = (E - 1 + f.bias) * (1 << f.mbits) + (static_cast<int>(r) - (1 << f.mbits));
  return idx > nmag - 1 ? nmag - 1 : idx;
}

bool shape_ok(int64_t N, int64_t K) {
  return N >= fp6::kTileN && K >= fp6::kTileK && N <= fp6::kMaxDim && K <= fp6::kMaxDim &&
         N % fp6::kTileN == 0 && K % fp6::kTileK == 0 && N * K <= fp6::kMaxNK;
}

// One 16 x 256 tile of codes (rows of `src` K apart) into one packed tile.
// Lane L = 16g + r owns row r, k = 32j + 8g + i (k-step j, element i).
void pack_tile(int format, const uint8_t* src, int64_t K, uint8_t* tile) {
  // Per lane: 4-bit words w4[j/4][lane][j%4]; 6-bit formats add 2-bit words
  // w2[lane][j/2], FP5 adds 1-bit words w1[lane][j/4].
  uint32_t w4[2][64][4];
  uint32_t w2[64][4];
  uint32_t w1[64][2];
  std::memset(w4, 0, sizeof(w4));
  std::memset(w2, 0, sizeof(w2));
  std::memset(w1, 0, sizeof(w1));
  static const int kE2M3Base[8] = {0, 1, 2, 3, 8, 9, 10, 11};
  for (int lane = 0; lane < 64; ++lane) {
    const int r = lane & 15, g = lane >> 4;
    const uint8_t* row = src + r * K;
    for (int j = 0; j < 8; ++j) {
      for (int i = 0; i < 8; ++i) {
        const uint32_t c = row[32 * j + 8 * g + i];
        const int p = 4 * (j & 1) + (i >> 1);  // e2m3: pair in the 2-bit word
        const int h = i & 1;                   // even / odd element of the pair
        const int slot = (i >> 1) + 4 * (i & 1);
        uint32_t& d4 = w4[j >> 2][lane][j & 3];
        switch (format) {
          case FPX_E3M2: {
            // Group G = i/4 at byte E = i%4: e2 and s at bits 4 and 7 of byte
            // E once the word is rotated right by rho = 4(j%2) + 2G; the
            // nibble in slot 2E + G (low nibbles: elements 0..3).
            const int G = i >> 2, E = i & 3, rho = 4 * (j & 1) + 2 * G;
            w2[lane][j >> 1] |= ((c >> 4) & 1u) << ((4 + 8 * E + rho) & 31);
            w2[lane][j >> 1] |= ((c >> 5) & 1u) << ((7 + 8 * E + rho) & 31);
            d4 |= (c & 0xFu) << (4 * (2 * E + G));
            break;
          }
          case FPX_E2M3: {
            const int b = kE2M3Base[p] + 16 * h;
            w2[lane][j >> 1] |= ((c >> 4) & 1u) << b;
            w2[lane][j >> 1] |= ((c >> 5) & 1u) << (b + 4);
            d4 |= (c & 0xFu) << (4 * slot);
            break;
          }
          case FPX_E2M2: {
            // As e3m2's 4-bit word; the sign at bit 7 of byte E once the
            // 1-bit word is rotated right by 2(j%4) + G.
            const int G = i >> 2, E = i & 3;
            w1[lane][j >> 2] |= ((c >> 4) & 1u) << ((7 + 8 * E + 2 * (j & 3) + G) & 31);
            d4 |= (c & 0xFu) << (4 * (2 * E + G));
            break;
          }
          default:  // FPX_E2M1: whole code, natural nibble order
            d4 |= (c & 0xFu) << (4 * i);
            break;
        }
      }
    }
  }
  // Little-endian words: x86-64 hosts store them in the required byte order.
  switch (format) {
    case FPX_E3M2:
    case FPX_E2M3:
      std::memcpy(tile, w2, sizeof(w2));
      std::memcpy(tile + 1024, w4, sizeof(w4));
      break;
    case FPX_E2M2:
      std::memcpy(tile, w4, sizeof(w4));
      std::memcpy(tile + 2048, w1, sizeof(w1));
      break;
    default:
      std::memcpy(tile, w4, sizeof(w4));
      break;
  }
}


// 2:4-sparse FP6: one tile = 16 rows x 512 dense k (4096 bytes).  For k-step
// j (64 dense k) and lane L = 16g + r, element i is kept weight i%2 of the
// dense group at offset 64j + 32(g%2) + 16(i/4) + 8(g/2) + 4((i%4)/2): the
// A-operand order of v_smfmac_f32_16x16x64_f16.  The 6-bit codes fill bytes
// [0, 3072) exactly as the dense packer fills an FP6 tile (lane, k-step j,
// element i); the 2-bit positions fill [3072, 4096): lane L's word j/2 at
// 3072 + 16L, bits 16(j%2) + 2i.
void pack_sparse_tile(const uint8_t* codes, const uint8_t* pos, int64_t half_k, uint8_t* tile) {
  uint8_t fp6[16 * 256];  // codes in (row, 32j + 8g + i) order, one FP6 tile
  uint32_t wp[64][4];
  std::memset(wp, 0, sizeof(wp));
  for (int r = 0; r < 16; ++r) {
    for (int j = 0; j < 8; ++j) {
      for (int g = 0; g < 4; ++g) {
        for (int i = 0; i < 8; ++i) {
          const int off = 64 * j + 32 * (g & 1) + 16 * (i >> 2) + 8 * (g >> 1) + 4 * ((i & 3) >> 1);
          const int64_t t2 = 2 * (off / 4) + (i & 1);     // kept index inside the tile's row
          const uint8_t c = codes[r * half_k + t2];
          const uint32_t p = pos[r * half_k + t2];
          fp6[r * 256 + 32 * j + 8 * g + i] = c;
          wp[16 * g + r][j >> 1] |= p << (16 * (j & 1) + 2 * i);
        }
      }
    }
  }
  pack_tile(FPX_E3M2, fp6, 256, tile);
  std::memcpy(tile + 3072, wp, sizeof(wp));
}

}  // namespace

extern "C" {

int fp6_pack_version(void) { return 3; }

const char* fp6_status_string(int status) {
  switch (status) {
    case FP6_OK: return "ok";
    case FP6_E_NULL: return "a required pointer is NULL";
    case FP6_E_SHAPE: return "shape outside the supported range (N%16, K%256, limits)";
    case FP6_E_ALIGN: return "a device pointer is misaligned";
    case FP6_E_CODE: return "a weight code does not fit the format's width";
    case FP6_E_SCALE: return "a scale is not finite or outside the format's range";
    case FP6_E_SIZE: return "a buffer size does not match, or the plan needs more than the static scratch";
    case FP6_E_HIP: return "a HIP runtime call or kernel launch failed";
    case FP6_E_VALUE: return "an input value or plan parameter is invalid";
    default: return "unknown status";
  }
}

int fpx_bits(int format) {
  const FormatInfo* f = format_info(format);
  return f ? f->bits : 0;
}

size_t fpx_packed_bytes(int format, int64_t N, int64_t K) {
  const FormatInfo* f = format_info(format);
  if (!f || !shape_ok(N, K)) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 8 * static_cast<size_t>(f->bits);
}

size_t fp6_packed_bytes(int64_t N, int64_t K) { return fpx_packed_bytes(FPX_E3M2, N, K); }

int fpx_quantize_rows(int format, const float* W, int64_t N, int64_t K, uint8_t* codes,
                      uint16_t* scales) {
  const FormatInfo* f = format_info(format);
  if (!f) return FP6_E_VALUE;
  if (!W || !codes || !scales) return FP6_E_NULL;
  if (N < 1 || K < 1 || N > fp6::kMaxDim || K > fp6::kMaxDim || N * K > fp6::kMaxNK)
    return FP6_E_SHAPE;
  const int sign_shift = f->bits - 1;
  for (int64_t n = 0; n < N; ++n) {
    const float* row = W + n * K;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      if (!std::isfinite(row[k])) return FP6_E_VALUE;
      const float a = std::fabs(row[k]);
      if (a > amax) amax = a;
    }
    const uint16_t sb = double_to_half_rne(static_cast<double>(amax) / f->vmax);
    const double s = half_bits_to_double(sb);
    if (!std::isfinite(s) || std::fabs(s) >= f->scale_limit) return FP6_E_SCALE;
    scales[n] = sb;
    uint8_t* out = codes + n * K;
    if (s == 0.0) {
      std::memset(out, 0, static_cast<size_t>(K));
      continue;
    }
    for (int64_t k = 0; k < K; ++k) {
      const double q = static_cast<double>(row[k]) / s;
      const int sign = std::signbit(row[k]) ? 1 : 0;
      out[k] = static_cast<uint8_t>((sign << sign_shift) | magnitude_index(*f, std::fabs(q)));
    }
  }
  return FP6_OK;
}

int fp6_quantize_rows(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
  return fpx_quantize_rows(FPX_E3M2, W, N, K, codes, scales);
}

int fpx_prepack(int format, const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                void* packed, size_t packed_bytes) {
  const FormatInfo* f = format_info(format);
  if (!f) return FP6_E_VALUE;
  if (!codes || !scales || !packed) return FP6_E_NULL;
  if (!shape_ok(N, K)) return FP6_E_SHAPE;
  if (packed_bytes != fpx_packed_bytes(format, N, K)) return FP6_E_SIZE;
  for (int64_t n = 0; n < N; ++n) {
    const double s = half_bits_to_double(scales[n]);
    if (!std::isfinite(s) || std::fabs(s) >= f->scale_limit) return FP6_E_SCALE;
  }
  const size_t total = static_cast<size_t>(N) * static_cast<size_t>(K);
  const uint32_t code_end = 1u << f->bits;
  for (size_t i = 0; i < total; ++i)
    if (codes[i] >= code_end) return FP6_E_CODE;

  uint8_t* out = static_cast<uint8_t*>(packed);
  // Layout v3 orders the tiles k-tile-major: tile (nb, kb) is tile number
  // kb * nblocks + nb.
  const int64_t kblocks = K / fp6::kTileK, nblocks = N / fp6::kTileN;
  const int64_t tile_bytes = 4096 / 8 * f->bits;
  for (int64_t kb = 0; kb < kblocks; ++kb)
    for (int64_t nb = 0; nb < nblocks; ++nb)
      pack_tile(format, codes + nb * fp6::kTileN * K + kb * fp6::kTileK, K,
                out + (kb * nblocks + nb) * tile_bytes);
  return FP6_OK;
}

int fp6_prepack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                void* packed, size_t packed_bytes) {
  return fpx_prepack(FPX_E3M2, codes, scales, N, K, packed, packed_bytes);
}

// ---------------------------------------------------------------------------
// 2:4-sparse FP6 (fp6s_*).
// ---------------------------------------------------------------------------
size_t fp6s_packed_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K) || K % 512) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 2;
}

int fp6s_prune_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes, uint8_t* pos,
                        uint16_t* scales) {
  if (!W || !codes || !pos || !scales) return FP6_E_NULL;
  if (N < 1 || K < 4 || K % 4 || N > fp6::kMaxDim || K > fp6::kMaxDim || N * K > fp6::kMaxNK)
    return FP6_E_SHAPE;
  const FormatInfo& f = kFormats[FPX_E3M2];
  std::vector<float> kept(static_cast<size_t>(K / 2));
  for (int64_t n = 0; n < N; ++n) {
    const float* row = W + n * K;
    uint8_t* prow = pos + n * (K / 2);
    float amax = 0.0f;
    for (int64_t t = 0; t < K / 4; ++t) {
      const float* w = row + 4 * t;
      for (int q = 0; q < 4; ++q)
        if (!std::isfinite(w[q])) return FP6_E_VALUE;
      // the two largest magnitudes, the lower index first among equals
      int a = 0;
      for (int q = 1; q < 4; ++q)
        if (std::fabs(w[q]) > std::fabs(w[a])) a = q;
      int b = a == 0 ? 1 : 0;
      for (int q = 0; q < 4; ++q)
        if (q != a && std::fabs(w[q]) > std::fabs(w[b])) b = q;
      const int lo = a < b ? a : b, hi = a < b ? b : a;
      prow[2 * t] = static_cast<uint8_t>(lo);
      prow[2 * t + 1] = static_cast<uint8_t>(hi);
      kept[2 * t] = w[lo];
      kept[2 * t + 1] = w[hi];
      amax = std::fmax(amax, std::fmax(std::fabs(w[lo]), std::fabs(w[hi])));
    }
    const uint16_t sb = double_to_half_rne(static_cast<double>(amax) / f.vmax);
    const double s = half_bits_to_double(sb);
    if (!std::isfinite(s) || std::fabs(s) >= f.scale_limit) return FP6_E_SCALE;
    scales[n] = sb;
    uint8_t* out = codes + n * (K / 2);
    for (int64_t k = 0; k < K / 2; ++k) {
      if (s == 0.0) { out[k] = 0; continue; }
      const double q = static_cast<double>(kept[k]) / s;
      const int sign = std::signbit(kept[k]) ? 1 : 0;
      out[k] = static_cast<uint8_t>((sign << 5) | magnitude_index(f, std::fabs(q)));
    }
  }
  return FP6_OK;
}

int fp6s_prepack(const uint8_t* codes, const uint8_t* pos, const uint16_t* scales, int64_t N,
                 int64_t K, void* packed, size_t packed_bytes) {
  if (!codes || !pos || !scales || !packed) return FP6_E_NULL;
  if (!shape_ok(N, K) || K % 512) return FP6_E_SHAPE;
  if (packed_bytes != fp6s_packed_bytes(N, K)) return FP6_E_SIZE;
  const FormatInfo& f = kFormats[FPX_E3M2];
  for (int64_t n = 0; n < N; ++n) {
    const double s = half_bits_to_double(scales[n]);
    if (!std::isfinite(s) || std::fabs(s) >= f.scale_limit) return FP6_E_SCALE;
  }
  const size_t half = static_cast<size_t>(N) * static_cast<size_t>(K / 2);
  for (size_t i = 0; i < half; ++i)
    if (codes[i] > 63) return FP6_E_CODE;
  for (size_t i = 0; i < half; i += 2)
    if (pos[i] >= pos[i + 1] || pos[i + 1] > 3) return FP6_E_VALUE;
  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t kblocks = K / 512;
  for (int64_t nb = 0; nb < N / 16; ++nb)
    for (int64_t kb = 0; kb < kblocks; ++kb) {
      const int64_t off = nb * 16 * (K / 2) + kb * 256;
      pack_sparse_tile(codes + off, pos + off, K / 2, out + (nb * kblocks + kb) * 4096);
    }
  return FP6_OK;
}

}  // extern "C"
