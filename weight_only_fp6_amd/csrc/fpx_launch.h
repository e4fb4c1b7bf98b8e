// Interface between the host dispatch (plan, workspace, argument checks) and
// the per-format kernel translation units of the FPx linear layer.  Each
// format's kernels are instantiated in a file of their own so that they
// compile in parallel; the dispatch reaches them through launch_format().
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fpx {

// Weight formats (the values of the C ABI's `format` argument).
enum Format : int { kFmtE3M2 = 0, kFmtE2M3 = 1, kFmtE2M2 = 2, kFmtE2M1 = 3, kNumFormats = 4 };

// Kernel configurations reachable through the `variant` argument.
enum class Kind { kAuto, kStream, kTiled, kKsplit, kKslice, kXlds, kTiledSk, kKring };
struct KernelCfg {
  Kind kind;
  int a, mb, d;  // stream: row blocks/wave, 16-col blocks/wave, ring depth; tiled: B = mb
};
constexpr KernelCfg kCfgs[] = {
    {Kind::kAuto, 0, 0, 0},    // 0: automatic
    {Kind::kStream, 1, 1, 4},  // 1: streaming, 1 row block per wave, 16 columns, ring depth 4
    {Kind::kStream, 1, 4, 2},  // 2: streaming, 1 row block per wave, 64 columns, ring depth 2
    {Kind::kStream, 2, 1, 4},  // 3: streaming, 2 row blocks per wave, 16 columns, ring depth 4
    {Kind::kStream, 4, 1, 2},  // 4: streaming, 4 row blocks per wave, 16 columns, ring depth 2
    {Kind::kTiled, 4, 4, 4},   // 5: tiled, 256 rows x 64 columns, 4 waves x 4 row blocks
    {Kind::kTiled, 4, 8, 4},   // 6: tiled, 256 rows x 128 columns, 4 waves x 4 row blocks
    {Kind::kStream, 1, 1, 8},  // 7: streaming, 1 row block per wave, 16 columns, ring depth 8
    {Kind::kStream, 2, 1, 6},  // 8: streaming, 2 row blocks per wave, 16 columns, ring depth 6
    {Kind::kKsplit, 1, 1, 8},  // 9: k-split persistent, M <= 16, K <= 8192 per K-split (X in registers)
    {Kind::kTiled, 2, 8, 8},   // 10: tiled, 256 rows x 128 columns, 8 waves x 2 row blocks
    {Kind::kTiled, 2, 4, 8},   // 11: tiled, 256 rows x 64 columns, 8 waves x 2 row blocks
    {Kind::kKsplit, 1, 1, 16}, // 12: k-split persistent with 16 waves per workgroup
    {Kind::kKslice, 1, 1, 16}, // 13: k-slice, 16 waves per row block, X streamed
    {Kind::kXlds, 2, 1, 4},    // 14: streaming + X in LDS, 2 row blocks/wave, ring 4, 4 waves
    {Kind::kXlds, 1, 1, 4},    // 15: streaming + X in LDS, 1 row block/wave, ring 4, 4 waves
    {Kind::kXlds, 2, 1, 8},    // 16: streaming + X in LDS, 2 row blocks/wave, ring 4, 8 waves
    {Kind::kTiled, 2, 4, 8},   // 17: tiled, 256 rows x 64 columns, 8 waves, whole-tile stages
    {Kind::kXlds, 1, 1, 4},    // 18: streaming + X in LDS, 1 row block/wave, ring 4, 8 waves
    {Kind::kXlds, 2, 2, 2},    // 19: streaming + X in LDS, 2 row blocks x 32 columns per wave, ring 2, 8 waves
    {Kind::kXlds, 2, 4, 2},    // 20: streaming + X in LDS, 2 row blocks x 64 columns per wave, ring 2, 8 waves
    {Kind::kXlds, 1, 2, 4},    // 21: streaming + X in LDS, 1 row block x 32 columns per wave, ring 4, 8 waves
    {Kind::kXlds, 1, 4, 2},    // 22: streaming + X in LDS, 1 row block x 64 columns per wave, ring 2, 8 waves
    {Kind::kTiled, 2, 8, 8},   // 23: tiled, 256 rows x 128 columns, 8 waves x 2 row blocks, weights staged in LDS
    {Kind::kTiled, 2, 4, 8},   // 24: tiled, 256 rows x 64 columns, 8 waves x 2 row blocks, weights staged in LDS
    {Kind::kTiledSk, 2, 8, 8}, // 25: tiled (as 10), stream-K: one workgroup per CU, equal (tile, half-tile) ranges
    {Kind::kKring, 1, 1, 8},   // 26: k-ring, M <= 16, K <= 8192, <= 8 row blocks per CU (X in registers)
};
constexpr int kNumVariants = sizeof(kCfgs) / sizeof(kCfgs[0]);
constexpr int kKsMaxTiles = 32;      // k-split kernels: K <= 8192
constexpr int kKsliceMaxTiles = 48;  // k-slice kernels: K <= 12288
constexpr int kKringMaxTiles = 32;   // k-ring kernel: K <= 8192 (4 k-tiles per wave)
constexpr int kKringMaxRows = 8;     // k-ring kernel: row blocks per workgroup

// One resolved launch: shapes, device pointers, the schedule and the
// split-K workspace (part/counters are null when splits == 1).
struct LaunchCtx {
  const void* X;
  const void* W;
  const void* S;
  void* Y;
  int64_t M, N, K;
  int variant;  // 1..kNumVariants-1
  int splits;
  float* part;
  unsigned* counters;
  int cus;
  hipStream_t stream;
};

// Enqueue the planned kernel(s) of one format; returns an fp6_status.
int launch_e3m2(const LaunchCtx& c);
int launch_e2m3(const LaunchCtx& c);
int launch_e2m2(const LaunchCtx& c);
int launch_e2m1(const LaunchCtx& c);
// Enqueue the de-quantisation export of one format (W16 fp16 [N][K]).
int dequant_e3m2(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s);
int dequant_e2m3(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s);
int dequant_e2m2(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s);
int dequant_e2m1(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s);

// 2:4-sparse FP6 (fp6s_*): kernel configurations of fp6s_linear_plan.
enum SparseVariant : int {
  kSpAuto = 0, kSpKslice = 1, kSpXlds1 = 2, kSpXlds2 = 3, kSpTiled4 = 4, kSpTiled8 = 5, kSpKsplit = 6,
  kSpXldsMB1 = 7, kSpXldsMB2 = 8, kSpKring = 9, kNumSpVariants = 10
};
constexpr int kSpKsliceMaxTiles = 16;  // k-slice: one 512-k tile per wave, 16 waves
constexpr int kSpKsplitMaxTiles = 8;   // k-split: one 512-k tile per wave and K-split, 8 waves
constexpr int kSpKsplitMaxRows = 8;    // k-split: row blocks per workgroup
constexpr int kSpKringMaxTiles = 16;   // k-ring: K <= 8192 (2 sparse tiles per wave)
int64_t sp_ksplit_rows_per_wg(int64_t N, int cus, int splits);
int launch_sparse(const LaunchCtx& c);  // c.variant is a SparseVariant
int dequant_sparse(const void* W, const void* S, void* W16, int64_t N, int64_t K, hipStream_t s);

}  // namespace fpx
