// Host side of the FP6 (e3m2) weight-only linear layer: status strings,
// size rules, the row quantiser and the offline packer (layout v1).
//
// Plain C++17, no HIP calls: everything here runs on the CPU.
//
// TC-FPx explainer (duicuo.cn), section "redesigning the kernel solution":
// weights are re-ordered before inference and packed into aligned words, and
// each 6-bit weight is split into power-of-two pieces (2 + 4 bits) so the GPU
// can rebuild it with a few bit operations.  The concrete bit positions below
// are this library's own design for 64-lane wavefronts (see fp6.h).

#include "fp6.h"
#include "fp6_limits.h"

#include <cmath>
#include <cstring>
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

// Nearest e3m2 magnitude index (0..31) of q >= 0, ties to the even index,
// saturating at 28.  e3m2 value = 2^(e-3) * (1 + m/4) for e >= 1 and
// m * 2^-4 for e == 0; the index is e*4 + m.
int e3m2_magnitude_index(double q) {
  if (!(q < 28.0)) return 31;               // also +inf
  if (q < 0.25) {                           // subnormal grid, spacing 2^-4
    return static_cast<int>(std::nearbyint(q * 16.0));  // 4 -> 0.25, the first normal
  }
  int E;
  const double f = std::frexp(q, &E);       // q = f * 2^E, f in [0.5, 1)
  double r = std::nearbyint(f * 8.0);       // 3 significant bits: r in 4..8
  if (r == 8.0) { r = 4.0; ++E; }
  // value = r/8 * 2^E = (4 + m)/4 * 2^(e-3)  =>  e = E + 2, m = r - 4
  const int idx = (E + 2) * 4 + (static_cast<int>(r) - 4);
  return idx > 31 ? 31 : idx;
}

bool shape_ok(int64_t N, int64_t K) {
  return N >= fp6::kTileN && K >= fp6::kTileK && N <= fp6::kMaxDim && K <= fp6::kMaxDim &&
         N % fp6::kTileN == 0 && K % fp6::kTileK == 0 && N * K <= fp6::kMaxNK;
}

}  // namespace

extern "C" {

int fp6_pack_version(void) { return 1; }

const char* fp6_status_string(int status) {
  switch (status) {
    case FP6_OK: return "ok";
    case FP6_E_NULL: return "a required pointer is NULL";
    case FP6_E_SHAPE: return "shape outside the supported range (N%16, K%256, limits)";
    case FP6_E_ALIGN: return "a device pointer is misaligned";
    case FP6_E_CODE: return "a weight code is larger than 63";
    case FP6_E_SCALE: return "a scale is not finite or has |s| >= 16";
    case FP6_E_SIZE: return "a buffer size does not match";
    case FP6_E_HIP: return "a HIP runtime call or kernel launch failed";
    case FP6_E_VALUE: return "an input value or plan parameter is invalid";
    default: return "unknown status";
  }
}

size_t fp6_packed_bytes(int64_t N, int64_t K) {
  if (!shape_ok(N, K)) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K) / 4 * 3;
}

int fp6_quantize_rows(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales) {
  if (!W || !codes || !scales) return FP6_E_NULL;
  if (N < 1 || K < 1 || N > fp6::kMaxDim || K > fp6::kMaxDim || N * K > fp6::kMaxNK)
    return FP6_E_SHAPE;
  for (int64_t n = 0; n < N; ++n) {
    const float* row = W + n * K;
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      if (!std::isfinite(row[k])) return FP6_E_VALUE;
      const float a = std::fabs(row[k]);
      if (a > amax) amax = a;
    }
    const uint16_t sb = double_to_half_rne(static_cast<double>(amax) / 28.0);
    const double s = half_bits_to_double(sb);
    if (!std::isfinite(s) || std::fabs(s) >= 16.0) return FP6_E_SCALE;
    scales[n] = sb;
    uint8_t* out = codes + n * K;
    if (s == 0.0) {
      std::memset(out, 0, static_cast<size_t>(K));
      continue;
    }
    for (int64_t k = 0; k < K; ++k) {
      const double q = static_cast<double>(row[k]) / s;
      const int sign = std::signbit(row[k]) ? 1 : 0;
      out[k] = static_cast<uint8_t>((sign << 5) | e3m2_magnitude_index(std::fabs(q)));
    }
  }
  return FP6_OK;
}

int fp6_prepack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                void* packed, size_t packed_bytes) {
  if (!codes || !scales || !packed) return FP6_E_NULL;
  if (!shape_ok(N, K)) return FP6_E_SHAPE;
  if (packed_bytes != fp6_packed_bytes(N, K)) return FP6_E_SIZE;
  for (int64_t n = 0; n < N; ++n) {
    const double s = half_bits_to_double(scales[n]);
    if (!std::isfinite(s) || std::fabs(s) >= 16.0) return FP6_E_SCALE;
  }
  const size_t total = static_cast<size_t>(N) * static_cast<size_t>(K);
  for (size_t i = 0; i < total; ++i)
    if (codes[i] > 63) return FP6_E_CODE;

  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t kblocks = K / fp6::kTileK;
  // One tile = 16 rows x 256 k -> 64 lanes x (4 two-bit words + 8 four-bit words).
  for (int64_t nb = 0; nb < N / fp6::kTileN; ++nb) {
    for (int64_t kb = 0; kb < kblocks; ++kb) {
      uint32_t w2[64][4];
      uint32_t w4[2][64][4];
      std::memset(w2, 0, sizeof(w2));
      std::memset(w4, 0, sizeof(w4));
      for (int lane = 0; lane < 64; ++lane) {
        const int r = lane & 15, g = lane >> 4;
        const uint8_t* src = codes + (nb * fp6::kTileN + r) * K + kb * fp6::kTileK;
        for (int j = 0; j < 8; ++j) {
          for (int i = 0; i < 8; ++i) {
            const uint32_t c = src[32 * j + 8 * g + i];
            const int p = 4 * (j & 1) + (i >> 1);
            const int h = i & 1;
            const int pos_e2 = (12 + 16 * h + 2 * p) & 31;
            const int pos_s = (15 + 16 * h + 2 * p) & 31;
            w2[lane][j >> 1] |= ((c >> 4) & 1u) << pos_e2;
            w2[lane][j >> 1] |= ((c >> 5) & 1u) << pos_s;
            const int slot = (i >> 1) + 4 * (i & 1);
            w4[j >> 2][lane][j & 3] |= (c & 0xFu) << (4 * slot);
          }
        }
      }
      uint8_t* tile = out + (nb * kblocks + kb) * fp6::kTileBytes;
      // Little-endian words: x86-64 hosts store them in the required byte order.
      std::memcpy(tile, w2, sizeof(w2));
      std::memcpy(tile + 1024, w4, sizeof(w4));
    }
  }
  return FP6_OK;
}

}  // extern "C"
