// Tile geometry and size limits shared by the host code and the kernels of
// the FP6 library (packed layout v3: 16 rows x 256 k per 3072-byte tile).
#pragma once
#include <stdint.h>

namespace fp6 {
constexpr int64_t kTileN = 16;
constexpr int64_t kTileK = 256;
constexpr int64_t kTileBytes = 3072;
constexpr int64_t kMaxDim = int64_t(1) << 24;
constexpr int64_t kMaxNK = int64_t(1) << 36;
}  // namespace fp6
